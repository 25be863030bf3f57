/*
 * trellis_micro.h -- microbenchmarks of libtrellis.so: the hardware ceilings that bound the
 * trellis-coded products on MI355X (gfx950).  They measure the machine, not the method:
 *
 *   - the cold HBM stream-read rate, the ceiling of the batch-1 products, which read each
 *     code byte once ("EXLR8" page, introduction: decode speed is bound by the bytes of
 *     weights read per token);
 *   - the issue cost of the vector instructions that decode a trellis state into its
 *     codebook value ("The escha W2 format, recovered and verified", "Codebook: cb=1 (MCG),
 *     verified": a 32-bit multiply, a mask/xor and an fp16 add per weight), alone and as
 *     whole per-tile decode sequences, which bound the batch-1 products when the decode
 *     takes longer than the code bytes take to arrive;
 *   - the issue rate of the matrix instructions the batched products use.
 *
 * Conventions as in trellis.h: device pointers, `stream` is a hipStream_t as void*, nothing
 * is allocated or synchronised, validation failures return a negative trellis_status before
 * anything is enqueued (message in trellis_last_error()).
 */
#ifndef TRELLIS_MICRO_H_
#define TRELLIS_MICRO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Vector-instruction kernels of trellis_micro_valu(). */
enum {
  TRELLIS_MICRO_V_ADD_U32 = 0,        /* v_add_u32                                          */
  TRELLIS_MICRO_V_MUL_LO_U32 = 1,     /* v_mul_lo_u32 (the hash's 32-bit multiply)          */
  TRELLIS_MICRO_V_MUL_U32_U24 = 2,    /* v_mul_u32_u24                                      */
  TRELLIS_MICRO_V_MAD_U32_U24 = 3,    /* v_mad_u32_u24                                      */
  TRELLIS_MICRO_V_MAD_U32_U16 = 4,    /* v_mad_u32_u16, high-half source (op_sel)           */
  TRELLIS_MICRO_V_MUL_LO_U16_SDWA = 5,/* v_mul_lo_u16, word-select source, high-half result */
  TRELLIS_MICRO_V_PK_MUL_LO_U16 = 6,  /* v_pk_mul_lo_u16                                    */
  TRELLIS_MICRO_V_BFE_U32 = 7,        /* v_bfe_u32 (window extraction)                      */
  TRELLIS_MICRO_V_ALIGNBIT_B32 = 8,   /* v_alignbit_b32 (funnel shift of two words)         */
  TRELLIS_MICRO_V_PERM_B32 = 9,       /* v_perm_b32                                         */
  TRELLIS_MICRO_V_BITOP3_B32 = 10,    /* v_bitop3_b32 (the hash's mask and xor in one)      */
  TRELLIS_MICRO_V_LSHRREV_B32 = 11,   /* v_lshrrev_b32                                      */
  TRELLIS_MICRO_V_ADD_F16_SDWA = 12,  /* v_add_f16 of a word's two halves (codebook sum)    */
  TRELLIS_MICRO_V_MUL_U32_U24_SDWA = 13, /* v_mul_u32_u24, word-select source               */
  TRELLIS_MICRO_V_FMA_F32 = 14,       /* v_fma_f32                                          */
  /* Whole per-tile decode of the products (one lane's four states of a 16x16 tile, K = 3):
   * the instructions that turn two code words into four hash words.  Counted per tile.  */
  TRELLIS_MICRO_DECODE_TILE = 100,    /* the products' sequence (funnel, extract, multiply, mask-xor) */
  TRELLIS_MICRO_DECODE_TILE_MFMA = 101,/* the same, each tile's words fed to one 16x16x32 fp16 MFMA */
  TRELLIS_MICRO_DECODE_TILE_U24 = 102 /* a 24-bit-multiply form of the same hash           */
};

/* Matrix-instruction kernels of trellis_micro_mfma(). */
enum {
  TRELLIS_MICRO_MFMA_F16_16X16X32 = 0,   /* v_mfma_f32_16x16x32_f16                        */
  TRELLIS_MICRO_MFMA_F16_32X32X16 = 1,   /* v_mfma_f32_32x32x16_f16                        */
  TRELLIS_MICRO_MFMA_F8_16X16X128 = 2,   /* v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3)       */
  TRELLIS_MICRO_MFMA_F8_32X32X64 = 3     /* v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3)        */
};

/* Stream-read `bytes` (a multiple of 16, >= 16) from `buf` with 16-byte loads by every CU
 * (`blocks` workgroups of 256 threads, 0 = 8 per CU), folding what it reads into one word
 * per thread of `sink` (uint32 [blocks * 256]; prevents the loads from being dropped).
 * `buf` must be 16-byte aligned.  Time the call with events around it: bytes / time is the
 * stream-read rate (cold when `buf` is far larger than the 256 MB Infinity Cache). */
int trellis_micro_stream_read(const void *buf, size_t bytes, int blocks, uint32_t *sink, void *stream);

/* Runs `iters` iterations of kernel `op` (TRELLIS_MICRO_V_* or TRELLIS_MICRO_DECODE_*) in
 * `waves_per_simd` (1..8) waves on each SIMD of every CU.  Per iteration a wave issues 64
 * instructions of the kind (8 independent chains), or 16 tile decodes.  Writes, per
 * workgroup (4 waves), the shader-clock cycles of its timed loop (s_memtime) to
 * cycles[wg] and the constant-rate (100 MHz) ticks to ticks[wg] (both uint64, [CUs *
 * waves_per_simd]); the clock is cycles / ticks * 100 MHz.  Per SIMD, a wave instruction
 * then costs cycles / (waves_per_simd * iters * 64) clocks (per tile: / 16).  sink: uint32
 * [CUs * waves_per_simd * 256].  Returns the number of workgroups launched, or < 0. */
int trellis_micro_valu(int op, int iters, int waves_per_simd, uint64_t *cycles, uint64_t *ticks, uint32_t *sink,
                       void *stream);

/* Runs `iters` iterations of 8 independent matrix instructions of kind `kind`
 * (TRELLIS_MICRO_MFMA_*) per wave, `waves_per_simd` (1..4) waves per SIMD on every CU.
 * cycles/ticks/sink as trellis_micro_valu (sink: float [workgroups * 256]).  Returns the
 * number of workgroups launched, or < 0.  Flops per instruction: 2*M*N*K of its shape. */
int trellis_micro_mfma(int kind, int iters, int waves_per_simd, uint64_t *cycles, uint64_t *ticks, float *sink,
                       void *stream);

/* Compute units of the current device (the micro kernels size their grids from it). */
int trellis_micro_cus(void);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_MICRO_H_ */
