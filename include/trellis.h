/*
 * trellis.h -- C ABI of libtrellis.so: products against EXL3-style trellis-coded weights
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *   - Storage ("The escha W2 format, recovered and verified", "Tensor mapping"): a layer
 *     y = x W with W [in, out] is stored as `code` int16 [in/16][out/16][16*K] (one packed
 *     16x16 tile per (i, j), input-tile index major), `rin` fp16 [in], `rout` fp16 [out]
 *     and the escha scale vectors `s_in` f32 [in], `s_out` f32 [out].
 *   - Decode (same page, "Bit layout" and "Codebook: cb=1 (MCG)"): each tile's 256 symbols
 *     take the circular 16-bit window that ends at the symbol's own K bits of the tile
 *     bitstream (32-bit words, most significant bit first, each word = two little-endian
 *     int16 halves); the state maps through v = s * 0xCBAC1FED, (v & 0x8FFF8FFF) ^
 *     0x3B603B60, value = fp16(lo) + fp16(hi) rounded to fp16; symbol s lands at tile row
 *     8*((s>>1)&1) + 2*((s>>3)&3) + (s&1), column 8*((s>>2)&1) + (s>>5)
 *     ("Escha-W2 runs on Metal", tile/permutation paragraph).
 *   - Forward ("Escha-W2 runs on Metal", reconstruction paragraph): su = rin*s_in,
 *     sv = rout*s_out, xh = had(x*su), y = had(xh @ W_hat) * sv, where had() applies the
 *     normalised Sylvester Hadamard H_128/sqrt(128) to each 128-block of the last axis.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise.  fp16 data is passed as
 *     uint16_t bit patterns.  All arrays are dense, row-major, with no padding.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every call
 *     only enqueues work on `stream`: it never allocates, frees or synchronises, and keeps
 *     no pointer after it returns.  Calls are thread-safe; the error string is per thread.
 *   - Validation happens on the host BEFORE anything is enqueued.  A failed check returns a
 *     negative trellis_status and sets trellis_last_error(); nothing is launched.  A launch
 *     failure returns TRELLIS_EHIP with the HIP error text.  No exception crosses the ABI.
 *   - Workspaces are owned by the caller, 256-byte aligned, and zero-filled before their
 *     first use.  Every workspace starts with the same reserved region: bytes [0, 256) are a
 *     header whose first uint32 is the ERROR WORD, and the next 64 KiB hold the small-batch
 *     products' counters, which each call leaves at zero again and no entry point leaves
 *     dirty.  So one zero-filled buffer, large enough for the largest request, serves any
 *     number of back-to-back calls of every entry point, in any order, on ONE stream.
 *     Calls that overlap in time (several streams) need separate workspaces.
 *   - The error word is sticky: kernels only OR bits into it (1: a routed id out of range
 *     or a table entry with an invalid K/cb was skipped; 2: a prefill workgroup's bounded
 *     wait for another ran out).  The caller reads it and clears it by writing 0 to the
 *     first 4 bytes of the workspace (any device fill, e.g. on the same stream).
 */
#ifndef TRELLIS_H_
#define TRELLIS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRELLIS_ABI_VERSION 2

typedef enum {
  TRELLIS_OK = 0,
  TRELLIS_EINVAL = -1,      /* bad size, K, cb, batch, side flag or NULL required pointer */
  TRELLIS_EALIGN = -2,      /* a pointer is not aligned as required */
  TRELLIS_EWORKSPACE = -3,  /* workspace NULL or smaller than trellis_workspace_bytes() */
  TRELLIS_EUNSUPPORTED = -4,/* valid request that this library does not implement */
  TRELLIS_EHIP = -5         /* a HIP runtime call failed; see trellis_last_error() */
} trellis_status;

/* One trellis-coded linear layer, y = x W, W [in_features, out_features].
 * code  : int16 [in/16][out/16][16*K], 16-byte aligned.
 * rin   : fp16 [in]  (EXL3 suh);  rout: fp16 [out] (EXL3 svh).
 * s_in  : f32 [in]  or NULL (= all ones);  s_out: f32 [out] or NULL (= all ones).
 * K in {2,3,4}; in and out multiples of 128.
 * cb = 1: the MCG codebook (fp16 values); cb = 2: the same values rounded to E4M3 (round to
 * nearest, ties to even, saturating), the EXLR8 format's codebook.
 * ("The escha W2 format, recovered and verified", "Tensor mapping": the config tensor
 *  [16, bits, cb, 1, in, out] fixes tile 16, K = bits, cb; "EXLR8" page, E4M3 paragraph.)
 * Every product takes either codebook per matrix (table entries may mix them);
 * trellis_gemm_fp8 requires cb = 2. */
typedef struct {
  const int16_t *code;
  const uint16_t *rin;
  const uint16_t *rout;
  const float *s_in;
  const float *s_out;
  int32_t K;
  int32_t in_features;
  int32_t out_features;
  int32_t cb;
} trellis_linear;

/* Operation ids for trellis_workspace_bytes(). */
enum { TRELLIS_OP_GEMV = 0, TRELLIS_OP_GEMM = 1, TRELLIS_OP_MOE_GEMV = 2, TRELLIS_OP_GEMM_FP8 = 3 };

int trellis_abi_version(void);

/* Text of the last error on the calling thread ("" if none).  Valid until the next call. */
const char *trellis_last_error(void);

/* Decode packed tiles to the codebook-domain matrix, bit-exact.
 * ("The escha W2 format ...", "Bit layout" and "Codebook"; "Escha-W2 runs on Metal",
 *  tile/permutation paragraph.)
 * code   : int16 [in/16][out/16][16*K], 16-byte aligned.
 * w_hat  : fp16 out [in][out] = W_hat (no Hadamard, no scales), 16-byte aligned.
 * states : NULL, or uint16 out [in/16][out/16][256]: each symbol's 16-bit trellis state in
 *          symbol order (for layout checks).
 * K in {2,3,4}; in, out multiples of 16. */
int trellis_decode_tiles(const int16_t *code, int K, int in_features, int out_features,
                         uint16_t *w_hat, uint16_t *states, void *stream);

/* Blockwise Hadamard-128 with a fused per-channel scale.
 * ("Escha-W2 runs on Metal", reconstruction paragraph: xh = had(x*su), y = had(y_pre)*sv.)
 * x   : [rows][n], fp32 if x_is_fp32 else fp16.       y: [rows][n], fp32 if y_is_fp32 else fp16.
 * r   : fp16 [n] or NULL (ones);  s: f32 [n] or NULL (ones).
 * post = 0: y = had(x * r * s)      (input side)
 * post = 1: y = had(x) * r * s      (output side)
 * had() is the normalised H_128/sqrt(128) on each consecutive 128-block; n % 128 == 0,
 * rows >= 0 (0 is a no-op).  x and y may alias exactly (in place). */
int had128_scale(const void *x, int x_is_fp32, int rows, int n, const uint16_t *r, const float *s,
                 int post, void *y, int y_is_fp32, void *stream);

/* Bytes of workspace needed by an op.  op = TRELLIS_OP_GEMV (batch_or_M = B),
 * TRELLIS_OP_GEMM or TRELLIS_OP_GEMM_FP8 (batch_or_M = M), TRELLIS_OP_MOE_GEMV (L = any entry of the uniform
 * table: only in/out are read, batch_or_M ignored, n_routed = n).  Host pointer L.
 * Returns 0 for invalid arguments. */
size_t trellis_workspace_bytes(int op, const trellis_linear *L, int batch_or_M, int n_routed);

/* Small-batch product y = had(had(x*su) @ W_hat) * sv.
 * ("Escha-W2 runs on Metal", reconstruction paragraph.)
 * L  : HOST pointer to the layer descriptor (its array pointers are device pointers).
 * x  : fp16 [B][in], y: fp16 out [B][out]; 1 <= B <= 8.  y must not overlap x.
 * ws : zero-filled device workspace of >= trellis_workspace_bytes(GEMV, L, B, 0) bytes.
 * One launch (the one-item case of trellis_gemv_list). */
int trellis_gemv(const trellis_linear *L, const uint16_t *x, int B, uint16_t *y,
                 void *ws, size_t ws_bytes, void *stream);

/* Several small-batch products in ONE launch: for each item p,
 *   y_p = had(had(x_p*su_p) @ W_hat_p) * sv_p           (the trellis_gemv definition)
 * Layers may differ in shape, K and codebook; the work of all of them is shared evenly by
 * every compute unit, and each output column block is finished by the last workgroup to
 * complete its share of it, so the whole list costs one launch.  Independent layers that
 * run back to back (a model's q/k/v projections, gate and up, or layers whose inputs are
 * ready together) take one call.
 * ("Escha-W2 runs on Metal", reconstruction paragraph, per layer.)
 * items : HOST array of n descriptors, 1 <= n <= TRELLIS_GEMV_LIST_MAX; each item's layer is
 *         checked as for trellis_gemv, x_p fp16 [B][in_p], y_p fp16 out [B][out_p].  No
 *         output may overlap another output or any input.
 * B     : 1..8 rows, the same for every item.
 * ws    : zero-filled device workspace of >= trellis_gemv_list_workspace_bytes(items, n, B)
 *         bytes (see the conventions above).
 * Returns TRELLIS_EUNSUPPORTED when the items have more than 16384 output column blocks
 * (128 columns each) together. */
#define TRELLIS_GEMV_LIST_MAX 8
typedef struct {
  trellis_linear L;
  const uint16_t *x;
  uint16_t *y;
} trellis_gemv_item;

/* Workspace bytes trellis_gemv_list needs (0 if the arguments are invalid or unsupported). */
size_t trellis_gemv_list_workspace_bytes(const trellis_gemv_item *items, int n, int B);

int trellis_gemv_list(const trellis_gemv_item *items, int n, int B, void *ws, size_t ws_bytes, void *stream);

/* trellis_gemv_list without a workspace argument, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and results, with the scratch (counters and partial sums) in a buffer of 32 MiB
 * that the library holds in device memory, one per device, for the life of the process.
 * Allocates nothing and calls no allocating routine.  Every call on a device shares that
 * device's buffer, so calls that overlap in time on one device (several streams or threads)
 * race and must not be made.  A request needing more scratch than the buffer holds is
 * rejected with TRELLIS_EUNSUPPORTED before anything is enqueued (a dense MLP step of three
 * 5120 <-> 17408 matrices needs about 1 MiB of it at batch 1, 8 MiB at batch 8). */
int trellis_gemv_list_noalloc(const trellis_gemv_item *items, int n, int B, void *stream);

/* Prefill product, same definition as trellis_gemv for M rows (M >= 1).
 * x: fp16 [M][in], y: fp16 out [M][out].
 * ws: zero-filled device workspace of >= trellis_workspace_bytes(GEMM, L, M, 0) bytes
 *     (holds the rotated activations after the reserved region).  Two launches. */
int trellis_gemm(const trellis_linear *L, const uint16_t *x, int M, uint16_t *y,
                 void *ws, size_t ws_bytes, void *stream);

/* Decode to E4M3 bytes (the cb = 2 weights): w8[16i + r][16j + c] = the E4M3 code of
 * tile (i, j)'s element (r, c), i.e. the MCG codebook value rounded to E4M3.  Bit-exact.
 * ("EXLR8" page, E4M3 paragraph: EXL3's decode followed by the E4M3 rounding.)
 * code: int16 [in/16][out/16][16*K], 16-byte aligned; w8: uint8 out [in][out], 16-byte
 * aligned.  in, out multiples of 16 (0 is a no-op). */
int trellis_decode_tiles_e4m3(const int16_t *code, int K, int in_features, int out_features, uint8_t *w8,
                              void *stream);

/* Prefill on the FP8 matrix cores ("EXLR8" page: the E4M3 weights feed FP8 matrix
 * multiplies).  L->cb must be 2.  With xh = had(x*su) per row:
 *   sc_row = max|xh_row| / 448,  q = e4m3(xh_row / sc_row) (nearest even, saturating),
 *   y = had(sc_row * (q @ W_hat)) * sv
 * (an all-zero row gives y = 0).  x: fp16 [M][in], y: fp16 out [M][out], both 16-byte
 * aligned.  ws: device workspace of >= trellis_workspace_bytes(
 * TRELLIS_OP_GEMM_FP8, L, M, 0) bytes, 256-byte aligned (holds the E4M3 activations and
 * row scales).  Three launches. */
int trellis_gemm_fp8(const trellis_linear *L, const uint16_t *x, int M, uint16_t *y,
                     void *ws, size_t ws_bytes, void *stream);

/* Routed-expert products for one token: for k in [0, n), with e = routed[k],
 *   y[k] = had(had(x_k * su_e) @ W_hat_e) * sv_e,
 * x_k = x (shared, x_per_expert = 0, fp16 [in]) or x + k*in (x_per_expert = 1, fp16 [n][in]).
 * ("EXLR8" page: routed experts with per-expert widths K2/K3/K4; a pointer table re-read
 *  every launch; one hidden-side rotation shared by all experts so the token is rotated
 *  once.)
 * experts     : DEVICE array of E descriptors (uniform in_features/out_features, per-entry
 *               K, per-entry pointers); re-read on every launch.
 * routed      : DEVICE int32 [n], entries in [0, E).
 * shared_side : -1 none; 0: the input-side vectors of every entry are replaced by
 *               (shared_r, shared_s); 1: the output-side vectors are.  shared_r is fp16,
 *               shared_s is f32 or NULL.
 * y           : fp16 out [n][out].
 * An entry that is out of range or has an invalid K produces a zero output row and sets bit
 * 1 of the error word (see the conventions above); check tables once with
 * trellis_validate_table().  One launch. */
int trellis_moe_gemv(const trellis_linear *experts, int E, const int32_t *routed, int n,
                     int in_features, int out_features, const uint16_t *x, int x_per_expert,
                     const uint16_t *shared_r, const float *shared_s, int shared_side,
                     uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace trellis_moe_mlp needs for n routed experts (0 for invalid sizes). */
size_t trellis_moe_mlp_workspace_bytes(int hidden, int inter, int halves, int n);

/* Routed-expert MLP of one token, fused:
 *   for k in [0, n), e = routed[k]:
 *     g_k = gate_e(x), u_k = up_e(x)                   [inter]
 *     a_k = silu(g_k) * u_k      (elementwise; silu(z) = z / (1 + e^-z))
 *   y = sum_k router_w[k] * down_e(a_k)                [hidden]
 * where every product is the trellis_gemv definition with that matrix's vectors.
 * ("EXLR8" page: the calibration paragraph defines the expert activation a; the
 *  width-manifest paragraph stores gate/up per "half" of 128 intermediate channels with its
 *  own width and down with one width per expert, reached through a pointer table re-read
 *  every launch; the shared-rotation paragraph makes the hidden-side vectors one per layer,
 *  so x is rotated once for every expert and, because the down outputs share sv, the
 *  weighted sum is taken before a single output rotation.)
 * gate_up : DEVICE table [E][2*halves]: entry e*2H + h is slice h of gate_e (hidden ->
 *           inter/H, output channels h*inter/H ...), entry e*2H + H + h slice h of up_e.
 *           halves = inter/128 gives the per-half layout, halves = 1 one width per matrix.
 *           Input-side vectors of the entries are ignored (shared ones used).
 * down    : DEVICE table [E] (inter -> hidden); output-side vectors ignored.
 * routed  : DEVICE int32 [n], ids in [0, E).  router_w: DEVICE f32 [n].
 * x       : fp16 [hidden].  r_hidden_in/s_hidden_in: the shared gate/up input vectors,
 *           r_hidden_out/s_hidden_out: the shared down output vectors (s may be NULL).
 * act     : optional fp16 out [n][inter] receiving a_k (NULL: kept in the workspace).
 * y       : fp16 out [hidden]; n = 0 writes zeros.
 * ws      : zero-filled device workspace of >= trellis_moe_mlp_workspace_bytes() bytes
 *           (see the conventions above).
 * Two launches (gate/up with the activation, then down with the weighted sum).  A routed id
 * out of range or an entry with an invalid K contributes zero and sets bit 1 of the error
 * word.  a_k is stored as fp16 and is the input of down_e. */
int trellis_moe_mlp(const trellis_linear *gate_up, const trellis_linear *down, int E, int halves,
                    const int32_t *routed, const float *router_w, int n, int hidden, int inter,
                    const uint16_t *x, const uint16_t *r_hidden_in, const float *s_hidden_in,
                    const uint16_t *r_hidden_out, const float *s_hidden_out, uint16_t *act,
                    uint16_t *y, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace trellis_encode_tiles needs for n_tiles tiles (1 MiB per tile: the
 * search's decisions), 0 for n_tiles < 0. */
size_t trellis_encode_workspace_bytes(int n_tiles);

/* Tail-biting Viterbi encoder (the encode side of the format): for each 16x16 tile of
 * target values, the path through the 16-bit-state trellis (each symbol adds K bits) whose
 * codebook values have the least squared error, packed as the decoder reads it.
 * ("EXLR8" page, tile-coding paragraph; its E4M3 paragraph for cb = 2, where the search
 *  scores the E4M3-rounded values.)  The circular constraint: a first pass with a free
 * start gives the best end state n1; its low 16-K bits O fix the wrap; the second pass
 * starts from states with high bits O and ends in states with low bits O, so the path
 * closes.  Ties go to the lowest state index.  Path costs are float32: each step adds
 * (x - value)^2 computed as one subtraction, one multiplication and one addition, each
 * rounded (no fused multiply-add).
 * targets: f32 [n_tiles][16][16] (row = input row r, column = output column c of the
 *          tile, in the codebook domain: rotated and scaled as the decoder's W_hat);
 * code   : int16 out [n_tiles][16K] (tile words; trellis_decode_tiles reads them back);
 * states : optional uint16 out [n_tiles][256], the path's states in symbol order;
 * ws     : device workspace of >= trellis_encode_workspace_bytes(n_tiles), 256-byte aligned.
 * Two launches: the search (one 1024-thread workgroup per tile) and the backtrack. */
int trellis_encode_tiles(const float *targets, int n_tiles, int K, int cb, int16_t *code, uint16_t *states,
                         void *ws, size_t ws_bytes, void *stream);

/* Host-side check of a HOST copy of an expert table: K, cb, sizes, alignment, non-NULL
 * pointers (rin/rout may be NULL on a side that will be shared).  Returns TRELLIS_OK or the
 * first failing status (with the entry index in trellis_last_error()). */
int trellis_validate_table(const trellis_linear *host_table, int E, int in_features,
                           int out_features, int shared_side);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_H_ */
