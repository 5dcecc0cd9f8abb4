/*
 * qmm.h -- C ABI of libqmm: the prefill matrix multiply ("MMQ") of llama.cpp-style
 * k-quant weights (q6_K, q4_K) against activations quantized to q8 blocks of 32,
 * on AMD Instinct MI355X (gfx950).
 *
 *   out[t][j] = sum over k of  weight[j][k] * activation[t][k]
 *
 * computed the way the engineering log "minfer / cuda_optimization_steps"
 * describes it (pages "48 - r45 - cp.async for the q6_K A-side staging",
 * "59 - r56 - q6_K A-side bundle: A cp.async + W_dsc f32 plane", "61 - r58 -
 * q4_K BT spec + cp.async-db2 transplant"): the activations are first quantized
 * by a prepass into q8 blocks with a scale pair (r45 section 1.1), the weights
 * are expanded once at registration into planes the kernel can copy without
 * arithmetic (r56 sections 2.2-2.3, r58 section 3.2), and the GEMM forms exact
 * integer dot products per 32-element block and applies the per-block scales in
 * binary32.
 *
 * Conventions for every entry point:
 *   - Return QMM_OK (0) on success or a negative QMM_E* code; qmm_last_error()
 *     then names the problem.  No entry point ever falls back to another path.
 *   - Every argument is validated before the first HIP call, so invalid calls
 *     fail identically on machines with and without a GPU.
 *   - "stream" is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously on it; pointers the caller passes must stay
 *     valid until that work completes.  The library keeps no caller pointer past
 *     the call.
 *   - Device pointers belong to the device that is current when the call is
 *     made; a weights handle is bound to the device current at registration and
 *     may only be used while that device is current.
 *   - Handles are immutable after registration: concurrent qmm_mmq calls on
 *     different streams may share one handle.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight block types. */
#define QMM_Q4_K 4 /* 144-byte blocks of 256 weights: f16 d, f16 dmin, 12 bytes of
                      6-bit scales and mins (8 sub-blocks of 32), 128 bytes of
                      4-bit codes; weight = d*scale*code - dmin*min
                      (r58 sections 2.2, 3.1). */
#define QMM_Q6_K 6 /* 210-byte blocks of 256 weights: ql[128] low 4 bits,
                      qh[64] high 2 bits, int8 scales[16] (one per 16 weights),
                      f16 d; weight = d*scale*(code - 32)
                      (r56 sections 1, 3.2; r58 section 3.2). */
#define QMM_Q4_K_PACKED 14 /* q4_K blocks (the same 144-byte input as QMM_Q4_K)
                      registered with the 4-bit codes kept two per byte in the
                      device plane, as the raw qs bytes hold them (r58 section
                      2.2): 0.5 instead of 1 byte per weight, unpacked by the
                      GEMM.  Results are bit-identical to QMM_Q4_K's. */

/* Return codes. */
#define QMM_OK 0
#define QMM_EINVAL (-1) /* bad argument: type, size, null or misaligned pointer */
#define QMM_ESHAPE (-2) /* buffers that do not belong together (qact vs handle) */
#define QMM_ENOMEM (-3) /* device memory could not be allocated; nothing leaked */
#define QMM_EHIP (-4)   /* a HIP runtime call or kernel launch failed */

/* Size limits (validated): 1 <= od <= QMM_MAX_OD, 256 <= id <= QMM_MAX_ID with
 * id % 256 == 0, 0 <= n_tok <= QMM_MAX_TOKENS.  n_tok == 0 is an empty batch:
 * qmm_qact_bytes gives 0, and qmm_quantize_activations and qmm_mmq (with
 * qact_bytes 0) return QMM_OK without touching any pointer or the device. */
#define QMM_MAX_OD (1 << 21)
#define QMM_MAX_ID (1 << 20)
#define QMM_MAX_TOKENS (1 << 20)

/* Compute units a launch plan (qmm_mmq_plan) may be asked for: 1 .. QMM_MAX_CUS. */
#define QMM_MAX_CUS 65536

/* Tokens are padded to a multiple of this many in the qact buffer. */
#define QMM_TOKEN_PAD 128

typedef struct qmm_weights qmm_weights;

typedef struct {
    int type;            /* QMM_Q4_K, QMM_Q4_K_PACKED or QMM_Q6_K */
    int64_t od;          /* output rows */
    int64_t id;          /* inner dimension */
    int64_t od_pad;      /* rows padded with zeros to the row tile */
    size_t raw_bytes;    /* od * (id/256) * (144 or 210): the k-quant bytes */
    size_t plane_bytes;  /* device memory the handle holds */
    size_t wd_offset;    /* byte offset of the d plane (q6_K; q4_K: == plane_bytes) */
    size_t sm_offset;    /* byte offset of the stage-record plane of scales, mins,
                            d and dmin (q4_K; q6_K: == plane_bytes) */
} qmm_info;

/*
 * qmm_register_weights -- copy one k-quant weight matrix to the device and
 * expand it once into the planes the GEMM reads (the registration-time planes
 * of r56 section 2.2 and r58 section 3.2; layout: see qmm_weights_export).
 *   type        QMM_Q4_K, QMM_Q4_K_PACKED (q4_K blocks, codes kept packed on
 *               the device) or QMM_Q6_K
 *   od, id      the weight is od rows of id weights; id % 256 == 0.  Any od >= 1
 *               (odd included) is valid: rows are padded with zeros internally.
 *   host_bytes  host memory, od rows * (id/256) blocks, row major, exactly
 *               nbytes = od * (id/256) * (144 for both q4_K types, 210 for
 *               q6_K) bytes.  Copied; the caller
 *               keeps ownership and may free it when the call returns.
 *   stream      the copy and the expansion run on it; the call returns after
 *               both completed (it synchronizes the stream).
 *   out         receives the handle; release with qmm_release_weights.
 * Errors: QMM_EINVAL (type, sizes, nullptrs, nbytes mismatch), QMM_ENOMEM (device
 * memory or the cap of qmm_set_memory_cap), QMM_EHIP.  On error *out is left NULL
 * and no device memory stays allocated.
 */
int qmm_register_weights(int type, int64_t od, int64_t id, const void *host_bytes,
                         size_t nbytes, void *stream, qmm_weights **out);

/* qmm_weights_info -- sizes of a handle.  QMM_EINVAL on null pointers. */
int qmm_weights_info(const qmm_weights *w, qmm_info *out);

/*
 * qmm_weights_export -- copy a handle's device planes to host memory, for
 * inspection and byte-exact tests (the r56 section 4 plane read-back gate).
 * host must hold exactly bytes = info.plane_bytes.  Synchronous.
 * Plane layout (R = od_pad/32 row blocks of 32 rows, nchunk = id/32, nsb =
 * id/256; rows od..od_pad-1 are zero everywhere):
 *   at 0          q6_K: int8 [R][nchunk][2][2][32][16]: the scale-folded weight
 *                 w = scale[k/16] * (code - 32) of (row j, k) as w = 64*hi + lo
 *                 (lo in [0, 63]), hi (plane index p = 0) and lo (p = 1) at byte
 *                 ((j/32*nchunk + k/32)*2 + p)*1024 + ((k%32)/16)*512
 *                 + (j%32)*16 + k%16
 *                 q4_K: int8 [R][nchunk][2][32][16]: the 4-bit code (0..15)
 *                 of (row j, k) at byte (j/32*nchunk + k/32)*1024
 *                 + ((k%32)/16)*512 + (j%32)*16 + k%16
 *                 q4_K packed: uint8 [R][nchunk][2][32][8]: the code of
 *                 (row j, k) in the low nibble (k%16 < 8) or the high nibble
 *                 (k%16 >= 8) of byte (j/32*nchunk + k/32)*512
 *                 + ((k%32)/16)*256 + (j%32)*8 + k%8
 *   at wd_offset  q6_K only: f32 [R][nsb][32]: d of (row j, super-block b) at
 *                 element (j/32*nsb + b)*32 + j%32
 *   at sm_offset  q4_K only (both q4_K types): [R][nchunk/4][1024 bytes], one
 *                 record per (row block, stage g of chunks 4g..4g+3) at byte
 *                 (j/32*nchunk/4 + g)*1024, each holding
 *                 +0    binary16 [32][4]: the 6-bit scale of (row j, chunk
 *                       4g + i) as an integer at element (j%32)*4 + i
 *                 +256  binary16 [2][32][4]: the 6-bit min of (row j, chunk
 *                       8b + 4h + i) of the stage's super-block b = g/2 as an
 *                       integer at element (h*32 + j%32)*4 + i
 *                 +768  f32 [2][32]: d*2^25 (part 0) and -dmin (part 1) of
 *                       (row j, super-block b) at element part*32 + j%32; both
 *                       exact in binary32, zeros stored as +0
 *                 (the two records of a super-block both hold its mins, d and
 *                 dmin)
 * Errors: QMM_EINVAL (null pointers, bytes mismatch), QMM_EHIP.
 */
int qmm_weights_export(const qmm_weights *w, void *host, size_t bytes);

/* qmm_release_weights -- free a handle's device memory.  Not safe while work
 * that uses the handle is still in flight: synchronize first.  NULL is a no-op. */
void qmm_release_weights(qmm_weights *w);

/*
 * qmm_set_memory_cap -- upper bound on the device memory (bytes) that all live
 * handles of this process may hold together; registration that would exceed
 * it fails with QMM_ENOMEM before allocating.  0 removes the cap (default).
 * For callers that budget HBM between several consumers.
 */
void qmm_set_memory_cap(size_t bytes);

/*
 * qmm_qact_bytes -- size of the quantized-activation buffer for n_tok tokens of
 * id activations: T_pad * id * 9 / 8 with T_pad = n_tok rounded up to
 * QMM_TOKEN_PAD.  Returns 0 for n_tok == 0 (an empty batch) and if n_tok or
 * id is out of range.
 */
size_t qmm_qact_bytes(int64_t n_tok, int64_t id);

/*
 * qmm_quantize_activations -- the quantize-transpose prepass (r45 section 1.1):
 * f32 activations -> q8 blocks of 32 with a scale pair (r45 section 2.3: 32
 * int8 values plus 4 bytes; r56 section 1: "d/ssum").
 *   x           device f32 [n_tok][id], row major, 16-byte aligned.  Values
 *               must be finite with |x| <= 2046 (so the scaled sum fits f16);
 *               other values give unspecified (but memory-safe) results.
 *   qact        device buffer of exactly qact_bytes = qmm_qact_bytes(n_tok, id)
 *               bytes, 16-byte aligned, fully overwritten.
 * Per token t and block c of 32 activations x_k:
 *   amax = max |x_k|;  dh = f16(amax / 127)   (binary32 division, f16 round to
 *   nearest even);  q_k = clamp(rint(x_k / dh), -127, 127) (binary32 division,
 *   round half to even) or 0 when dh == 0;  s = f16(dh * sum q_k).
 * Layout of qact (T_pad tokens; tokens >= n_tok are all zero; nchunk = id/32):
 *   q plane at byte 0, 1024-byte fragments per (32-token block tb, chunk c):
 *     q of (t, k) at ((t/32)*nchunk + k/32)*1024 + ((k%32)/16)*512
 *                    + (t%32)*16 + k%16
 *   scale plane at byte T_pad*id, 128 bytes per (tb, c):
 *     (dh, s) of (t, c) at T_pad*id + ((t/32)*nchunk + c)*128 + (t%32)*4,
 *     two little-endian binary16 values, dh first.
 * Errors: QMM_EINVAL (sizes, null/misaligned pointers, qact_bytes mismatch),
 * QMM_EHIP.
 */
int qmm_quantize_activations(const float *x, int64_t n_tok, int64_t id, void *qact,
                             size_t qact_bytes, void *stream);

/*
 * qmm_mmq -- the GEMM: out[t][j] = sum over 32-blocks c of
 *   q6_K: sum over the block's two 16-groups g of d*sc_g*dh_c*D16_g
 *   q4_K: d*sc_c*dh_c*D32_c - dmin*min_c*s_c
 * with D the exact integer dot of the weight codes (q6_K: code - 32) and the q8
 * codes over the group (r56 section 2.2 for the q6_K d*sc pairs).  The integer
 * parts are exact; the scales are applied and summed in binary32 (error within
 * 1e-4 of the sum of the terms' magnitudes).
 *   w           handle from qmm_register_weights (current device = its device)
 *   qact        buffer written by qmm_quantize_activations for these n_tok and
 *               the handle's id; qact_bytes must equal qmm_qact_bytes(n_tok,
 *               id) or the call fails with QMM_ESHAPE.  16-byte aligned.
 *   out         device f32 [n_tok][od], row major, 4-byte aligned; every element
 *               is overwritten (no accumulation), nothing outside is written.
 * When the output tiles fill the GPU's compute units a whole number of times
 * plus a small remainder, the remainder's tiles are split along the inner
 * dimension into partial sums that a second kernel adds in a fixed order.  Their
 * scratch is one device buffer per (device, stream) of 64 KiB per compute unit
 * (16 MiB on MI355X), allocated with hipMalloc by the first call on that stream
 * that needs it and kept until qmm_stream_release or the end of the process;
 * calls on one stream share it in stream order.  Synchronize a stream before destroying it if an MMQ on it
 * may still run.  Results are deterministic: the same call gives the same bits.
 * Errors: QMM_EINVAL (also for a shape whose tiles exceed one launch: n_tok * od
 * beyond about 6.9e10, i.e. an output of 275 GB), QMM_ESHAPE, QMM_ENOMEM (the
 * scratch), QMM_EHIP.
 */
int qmm_mmq(const qmm_weights *w, const void *qact, size_t qact_bytes, int64_t n_tok,
            float *out, void *stream);

/*
 * qmm_stream_release -- give back the device memory qmm_mmq keeps for `stream`
 * (the tail-partials scratch above, on every device it was allocated for), for
 * callers that create and destroy streams: call it before destroying the
 * stream.  It synchronizes `stream` first (an MMQ on it may still read the
 * partials), then frees; a later qmm_mmq on the same stream allocates again.
 *   freed_bytes  NULL, or receives the bytes freed (0 if the stream held none).
 * A stream that holds nothing returns QMM_OK without any HIP call.  Not safe
 * concurrently with a qmm_mmq on the same stream from another thread.
 * Errors: QMM_EHIP (the stream's synchronization or the free failed; what was
 * not freed stays held and *freed_bytes counts what was).
 */
int qmm_stream_release(void *stream, size_t *freed_bytes);

/*
 * qmm_mmq_noalloc -- qmm_mmq for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, validation, kernels and results (bit for bit)
 * as qmm_mmq; it calls no hipMalloc, hipFree or other allocating routine.  The
 * tail partials (see qmm_mmq) live in a static device array of 16 MiB that
 * every GPU the library runs on holds until the process ends; its address is
 * looked up (hipGetSymbolAddress) on the first call on each device.
 *   - Every call on one GPU shares that GPU's array and leaves the last call's
 *     partials in it: calls that may overlap on one GPU (different streams
 *     without ordering between them) race.  Calls on one stream are ordered.
 *   - Nothing in the array needs clearing: each partial is written whole
 *     before it is read.
 *   - A launch that needs more than 16 MiB of partials (only on GPUs with more
 *     than 256 compute units) fails with QMM_EINVAL before any launch.
 * Errors: as qmm_mmq, without QMM_ENOMEM.
 */
int qmm_mmq_noalloc(const qmm_weights *w, const void *qact, size_t qact_bytes, int64_t n_tok,
                    float *out, void *stream);

/* The launch plan of one MMQ (qmm_mmq, qmm_mmq_noalloc): how its output tiles
 * map onto work-groups on a GPU of a given size, and the tail partials it needs.
 * The slots are the work-groups resident at once (per_cu per compute unit).  The
 * tiles of the whole waves, rounded down to whole row tiles (dp_row_tiles of
 * them, all tokens), run one work-group each.  The remaining row tiles' tiles
 * are split along the inner dimension into `split` slices of whole super-blocks,
 * computed by separate work-groups as f32 partial tiles that a second kernel
 * adds, when they form a partial wave: after at most one full wave (none
 * included: a launch filling at most half the GPU splits every tile), or, with
 * one or two work-groups per compute unit, a last wave of at most a quarter of
 * the slots behind several full ones -- and when there are at least two slices
 * to make (every wave group of a slice keeps a super-block). */
typedef struct {
    int64_t work_groups;   /* work-groups of the MMQ launch (0: an empty batch) */
    size_t scratch_bytes;  /* tail partials the call needs, n_tail * split partial
                              tiles of f32 (0: none); qmm_mmq_noalloc refuses a
                              call that needs more than its 16 MiB */
    int32_t threads;       /* threads per work-group */
    int32_t many;          /* 1: the many-tile geometry (several work-groups per
                              compute unit); 0: the few-tile one */
    int32_t tile_rows;     /* output rows per tile */
    int32_t tile_tokens;   /* tokens per tile */
    int32_t k_groups;      /* wave groups per work-group, each taking its share
                              of the work-group's super-blocks */
    int32_t per_cu;        /* work-groups resident per compute unit */
    int32_t row_tiles;     /* tiles covering the od rows ... */
    int32_t tok_tiles;     /* ... and the n_tok tokens */
    int32_t dp_row_tiles;  /* row tiles computed whole (== row_tiles without a tail) */
    int32_t n_tail;        /* tiles split along the inner dimension:
                              (row_tiles - dp_row_tiles) * tok_tiles */
    int32_t split;         /* slices per tail tile (1: no tail) */
    int32_t nsb;           /* super-blocks along the inner dimension, id / 256 */
} qmm_plan;

/*
 * qmm_mmq_plan -- the plan qmm_mmq follows for a handle of this type, od and id
 * at n_tok tokens on a GPU with num_cus compute units (the device attribute
 * hipDeviceAttributeMultiprocessorCount; 256 on MI355X).  Host arithmetic only:
 * no HIP call, no device needed.  For callers that size work ahead, e.g. that
 * check that a qmm_mmq_noalloc call fits its scratch (scratch_bytes).
 *   type, od, id, n_tok  as for qmm_register_weights and qmm_mmq
 *   num_cus     1 .. QMM_MAX_CUS
 *   out         receives the plan (zeroed, nsb set, for n_tok == 0)
 * Errors: QMM_EINVAL (arguments out of range, as the other entry points check
 * them; a shape whose tiles exceed one launch).
 */
int qmm_mmq_plan(int type, int64_t od, int64_t id, int64_t n_tok, int num_cus, qmm_plan *out);

/*
 * qmm_mmq_plan_work -- what work-group wg (0 <= wg < plan->work_groups) of a
 * plan's MMQ launch computes, by the kernel's own mapping: the tile of row tile
 * *row_tile (rows tile_rows * row_tile ...) and token tile *tok_tile, over
 * super-blocks [*sb_begin, *sb_end) of the inner dimension (all nsb of them for
 * a whole tile).  Host arithmetic only.  For inspection and tests of the plan.
 * Errors: QMM_EINVAL (NULL pointers, wg out of range, a plan whose fields do
 * not fit together).
 */
int qmm_mmq_plan_work(const qmm_plan *plan, int64_t wg, int32_t *row_tile, int32_t *tok_tile,
                      int32_t *sb_begin, int32_t *sb_end);

/* qmm_last_error -- message for the calling thread's last failed call ("" if
 * none).  Valid until the thread's next call into the library. */
const char *qmm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
