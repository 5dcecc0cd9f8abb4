/*
 * oracle.h -- plain CPU oracle for the q4_K / q6_K x q8 prefill matrix multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links or
 * calls this code; only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * Sources (the pages are the engineering log "minfer / cuda_optimization_steps"):
 *   [r56]  "59 - r56 - q6_K A-side bundle: A cp.async + W_dsc f32 plane (LANDED)",
 *          sections 1, 2.2, 2.3 and 3.2 (q6_K byte offsets ql/qh/scales/d, the
 *          d*sc pair per (chunk,row), exact f16->f32 and one f32 multiply).
 *   [r58]  "61 - r58 - q4_K BT spec + cp.async-db2 transplant (REVERTED)",
 *          sections 2.2, 3.1, 3.2 (q4_K 144-byte block, qs at byte 16, the
 *          get_scale_min_k4 6-bit scale/min unpack, q6_K value = q - 32).
 *   [r45]  "48 - r45 - cp.async for the q6_K A-side staging (REVERTED)",
 *          sections 1.1, 2.3 (q8 activation block: 32 int8 + a 4-byte scale
 *          pair, produced by a quantize-transpose prepass).
 * Where the pages leave a step open (element bit layouts inside the blocks, the
 * rounding of the activation quantizer, what "sum" means in the scale pair) the
 * readings used are the ones listed in the functions below; each is the public
 * llama.cpp ("ggml") k-quant / q8_1 convention restated in prose.
 *
 * Parity unpinned: the element bit layouts inside the q6_K ql/qh bytes, the q4_K
 * qs nibbles and the q4_K 12-byte scale/min packing are pinned by the tests only
 * to their restatement here (literal spot positions and a bit bijection); no
 * llama.cpp decoder or GGUF fixture is available to compare against.
 */
#ifndef QMM_ORACLE_H
#define QMM_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_Q4_K = 4, ORACLE_Q6_K = 6 };

/* IEEE binary16 <-> binary32/64.  f16 -> f32/f64 is exact.  f32 -> f16 rounds
 * to nearest, ties to even, with subnormals and overflow to infinity.        */
double   oracle_f16_to_f64(uint16_t h);
float    oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float f);

/* O1, q6_K decode.  raw: od rows x (id/256) blocks of 210 bytes, row major.
 *   w  [od][id]     : q - 32, in [-32, 31]
 *   sc [od][id/16]  : signed 8-bit scale of each 16-weight group
 *   d  [od][id/256] : the block's f16 super-scale, decoded exactly to f32  */
void oracle_decode_q6k(const uint8_t *raw, int64_t od, int64_t id,
                       int8_t *w, int8_t *sc, float *d);

/* O1, q4_K decode.  raw: od rows x (id/256) blocks of 144 bytes.
 *   w   [od][id]     : 4-bit code in [0, 15]
 *   sc  [od][id/32]  : 6-bit scale of each 32-weight sub-block
 *   mn  [od][id/32]  : 6-bit min of each 32-weight sub-block
 *   d, dmin [od][id/256]                                              */
void oracle_decode_q4k(const uint8_t *raw, int64_t od, int64_t id,
                       uint8_t *w, uint8_t *sc, uint8_t *mn, float *d, float *dmin);

/* O2, activation quantization to q8 blocks of 32.
 *   x  [n_tok][id] f32 (finite, |x| <= 2046)
 *   q  [n_tok][id] int8 in [-127, 127]
 *   dh [n_tok][id/32], s [n_tok][id/32] : binary16 bit patterns
 * Returns 0, or -1 if an input is not finite or exceeds the range.          */
int oracle_quantize(const float *x, int64_t n_tok, int64_t id,
                    int8_t *q, uint16_t *dh, uint16_t *s);

/* O3, integer dots.  q6_K: D16 [n_tok][od][id/16] per 16-group, and the
 * scale-folded J [n_tok][od][id/32] = sc_even*D16_even + sc_odd*D16_odd.
 * q4_K: D32 [n_tok][od][id/32].  Any output pointer may be NULL.            */
void oracle_dots_q6k(const uint8_t *raw, int64_t od, int64_t id,
                     const int8_t *q, int64_t n_tok, int32_t *D16, int32_t *J);
void oracle_dots_q4k(const uint8_t *raw, int64_t od, int64_t id,
                     const int8_t *q, int64_t n_tok, int32_t *D32);

/* O4, the result.  out[t][j] and A[t][j] = sum of |term| over every term of the
 * sum, both in f64.  Returns 0, or -1 on a bad type / shape.               */
int oracle_mmq(int type, const uint8_t *raw, int64_t od, int64_t id,
               const int8_t *q, const uint16_t *dh, const uint16_t *s,
               int64_t n_tok, double *out, double *A);

/* O4 at chosen (t, j) pairs only: out[i], A[i] for t = ts[i], j = js[i].     */
int oracle_mmq_at(int type, const uint8_t *raw, int64_t od, int64_t id,
                  const int8_t *q, const uint16_t *dh, const uint16_t *s,
                  int64_t n_tok, int64_t n, const int64_t *ts, const int64_t *js,
                  double *out, double *A);

/* O4 restricted to weight rows [j0, j1): out/A are [n_tok][j1 - j0].        */
int oracle_mmq_rows(int type, const uint8_t *raw, int64_t od, int64_t id,
                    const int8_t *q, const uint16_t *dh, const uint16_t *s,
                    int64_t n_tok, int64_t j0, int64_t j1, double *out, double *A);

#ifdef __cplusplus
}
#endif
#endif
