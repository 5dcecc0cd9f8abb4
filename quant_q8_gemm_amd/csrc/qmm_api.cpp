// qmm_api.cpp -- the C ABI declared in include/qmm.h: argument validation (all of
// it before the first HIP call), weight-handle lifetime, device-memory
// accounting, and the launches.  No compute happens here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qmm.h"
#include "qmm_internal.h"

struct qmm_weights {
  qmm::Planes p;
  int device;
  size_t raw_bytes;
  size_t plane_bytes;
  size_t wd_offset;
  size_t sm_offset;
  void* alloc;  // one device allocation holding every plane
};

namespace {

thread_local std::string g_last_error;
std::atomic<size_t> g_held{0};  // device bytes held by live handles
std::atomic<size_t> g_cap{0};   // 0 = no cap

// Scratch for the MMQ's tail partials: one buffer per (device, stream), of the
// largest size any call can need on that device (64 KiB per compute unit).
// Calls on one stream run in order, so they share it; it lives until
// qmm_stream_release(stream) or the process ends.
struct Scratch {
  int device;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};
std::mutex g_scratch_mu;
std::vector<Scratch> g_scratch;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(QMM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

void ok() { g_last_error.clear(); }

size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

size_t block_bytes(int type) { return qmm::is_q4k(type) ? 144 : 210; }

const char* type_name(int type) {
  return type == QMM_Q6_K ? "q6_K" : type == QMM_Q4_K ? "q4_K" : "q4_K (codes packed)";
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_id(int64_t id) {
  if (id < 256 || id > QMM_MAX_ID || id % 256 != 0)
    return fail(QMM_EINVAL, "id must be a multiple of 256 in [256, %d], got %lld", QMM_MAX_ID,
                (long long)id);
  return QMM_OK;
}

// n_tok == 0 is an empty batch: valid, and the call does nothing
int check_tokens(int64_t n_tok) {
  if (n_tok < 0 || n_tok > QMM_MAX_TOKENS)
    return fail(QMM_EINVAL, "n_tok must be in [0, %d], got %lld", QMM_MAX_TOKENS, (long long)n_tok);
  return QMM_OK;
}

int64_t token_pad(int64_t n_tok) { return (n_tok + qmm::kTokenPad - 1) / qmm::kTokenPad * qmm::kTokenPad; }

int check_type(int type) {
  if (type != QMM_Q4_K && type != QMM_Q4_K_PACKED && type != QMM_Q6_K)
    return fail(QMM_EINVAL, "type must be QMM_Q4_K (%d), QMM_Q4_K_PACKED (%d) or QMM_Q6_K (%d), got %d",
                QMM_Q4_K, QMM_Q4_K_PACKED, QMM_Q6_K, type);
  return QMM_OK;
}

int check_od(int64_t od) {
  if (od < 1 || od > QMM_MAX_OD)
    return fail(QMM_EINVAL, "od must be in [1, %d], got %lld", QMM_MAX_OD, (long long)od);
  return QMM_OK;
}

// The geometry part of a handle's planes (no memory): what the plan needs.
qmm::Planes plane_shape(int type, int64_t od, int64_t id) {
  qmm::Planes p{};
  p.type = type;
  p.od = od;
  p.id = id;
  p.od_pad = (int64_t)round_up((size_t)od, qmm::kRowPad);
  p.nsb = id / 256;
  p.nchunk = id / 32;
  return p;
}

// one-dimensional launch: work-groups x threads must stay below 2^32
int check_launch(const qmm::MmqPlan& plan, int64_t n_tok, int64_t od, int num_cus) {
  if ((uint64_t)plan.work_groups * (uint64_t)plan.threads >= (1ull << 32))
    return fail(QMM_EINVAL, "n_tok=%lld x od=%lld needs %lld work-groups, more than one launch holds",
                (long long)n_tok, (long long)od, (long long)plan.work_groups);
  if (plan.scratch_bytes > qmm::mmq_scratch_max_bytes(num_cus))
    return fail(QMM_EINVAL, "internal: tail scratch exceeds its bound");
  return QMM_OK;
}

}  // namespace

extern "C" {

const char* qmm_last_error(void) { return g_last_error.c_str(); }

void qmm_set_memory_cap(size_t bytes) { g_cap.store(bytes); }

size_t qmm_qact_bytes(int64_t n_tok, int64_t id) {
  if (n_tok < 0 || n_tok > QMM_MAX_TOKENS || id < 256 || id > QMM_MAX_ID || id % 256 != 0) return 0;
  return (size_t)token_pad(n_tok) * (size_t)id / 8 * 9;
}

int qmm_register_weights(int type, int64_t od, int64_t id, const void* host_bytes, size_t nbytes,
                         void* stream, qmm_weights** out) {
  if (out == nullptr) return fail(QMM_EINVAL, "out is NULL");
  *out = nullptr;
  if (int rc = check_type(type)) return rc;
  if (int rc = check_od(od)) return rc;
  if (int rc = check_id(id)) return rc;
  if (host_bytes == nullptr) return fail(QMM_EINVAL, "host_bytes is NULL");
  const size_t expect = (size_t)od * (size_t)(id / 256) * block_bytes(type);
  if (nbytes != expect)
    return fail(QMM_EINVAL, "nbytes %zu != od*(id/256)*%zu = %zu", nbytes, block_bytes(type), expect);

  qmm::Planes p = plane_shape(type, od, id);
  // q6_K: codes, d; q4_K: codes, stage records (one of the last two is empty)
  const size_t off_wd = round_up(qmm::wq_bytes(type, p.od_pad, id), 256);
  const size_t off_sm = off_wd + round_up(qmm::wd_bytes(type, p.od_pad, id), 256);
  const size_t plane_bytes = off_sm + round_up(qmm::wsm_bytes(type, p.od_pad, id), 256);
  // reserve the bytes against the cap before allocating, atomically, so that
  // registrations on several threads cannot overshoot it together; every
  // failure below gives them back
  const size_t cap = g_cap.load();
  size_t held = g_held.load();
  do {
    if (cap != 0 && held + plane_bytes > cap)
      return fail(QMM_ENOMEM, "registration needs %zu device bytes; cap %zu, held %zu", plane_bytes,
                  cap, held);
  } while (!g_held.compare_exchange_weak(held, held + plane_bytes));

  // ---- first HIP call below this line ----
  hipStream_t s = (hipStream_t)stream;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    g_held -= plane_bytes;
    return fail_hip(e, "hipGetDevice");
  }
  void* alloc = nullptr;
  void* raw = nullptr;
  e = hipMalloc(&alloc, plane_bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    g_held -= plane_bytes;
    return e == hipErrorOutOfMemory ? fail(QMM_ENOMEM, "hipMalloc(%zu) failed: out of memory", plane_bytes)
                                    : fail_hip(e, "hipMalloc(planes)");
  }
  e = hipMalloc(&raw, nbytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(alloc);
    g_held -= plane_bytes;
    return e == hipErrorOutOfMemory ? fail(QMM_ENOMEM, "hipMalloc(%zu) failed: out of memory", nbytes)
                                    : fail_hip(e, "hipMalloc(raw)");
  }
  p.wq = (int8_t*)alloc;
  p.wd = qmm::is_q4k(type) ? nullptr : (float*)((char*)alloc + off_wd);
  p.wsm = qmm::is_q4k(type) ? (uint8_t*)alloc + off_sm : nullptr;
  int rc = QMM_OK;
  if ((e = hipMemcpyAsync(raw, host_bytes, nbytes, hipMemcpyHostToDevice, s)) != hipSuccess)
    rc = fail_hip(e, "hipMemcpyAsync(weights)");
  else if ((e = qmm::launch_repack((const uint8_t*)raw, p, s)) != hipSuccess)
    rc = fail_hip(e, "repack launch");
  else if ((e = hipStreamSynchronize(s)) != hipSuccess)
    rc = fail_hip(e, "hipStreamSynchronize(registration)");
  (void)hipFree(raw);
  if (rc != QMM_OK) {
    (void)hipFree(alloc);
    g_held -= plane_bytes;
    return rc;
  }
  qmm_weights* w = new qmm_weights;
  w->p = p;
  w->device = device;
  w->raw_bytes = nbytes;
  w->plane_bytes = plane_bytes;
  w->wd_offset = qmm::is_q4k(type) ? plane_bytes : off_wd;
  w->sm_offset = qmm::is_q4k(type) ? off_sm : plane_bytes;
  w->alloc = alloc;
  if (getenv("QMM_LOG") != nullptr)
    fprintf(stderr, "qmm: registered %s od=%lld id=%lld od_pad=%lld raw=%zu planes=%zu device=%d\n",
            type_name(type), (long long)od, (long long)id,
            (long long)p.od_pad, nbytes, plane_bytes, device);
  *out = w;
  ok();
  return QMM_OK;
}

int qmm_weights_info(const qmm_weights* w, qmm_info* out) {
  if (w == nullptr || out == nullptr) return fail(QMM_EINVAL, "NULL handle or info pointer");
  out->type = w->p.type;
  out->od = w->p.od;
  out->id = w->p.id;
  out->od_pad = w->p.od_pad;
  out->raw_bytes = w->raw_bytes;
  out->plane_bytes = w->plane_bytes;
  out->wd_offset = w->wd_offset;
  out->sm_offset = w->sm_offset;
  ok();
  return QMM_OK;
}

int qmm_weights_export(const qmm_weights* w, void* host, size_t bytes) {
  if (w == nullptr || host == nullptr) return fail(QMM_EINVAL, "NULL handle or host pointer");
  if (bytes != w->plane_bytes)
    return fail(QMM_EINVAL, "bytes %zu != plane_bytes %zu", bytes, w->plane_bytes);
  int prev = -1;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (prev != w->device && (e = hipSetDevice(w->device)) != hipSuccess) return fail_hip(e, "hipSetDevice");
  e = hipMemcpy(host, w->alloc, bytes, hipMemcpyDeviceToHost);
  if (prev != w->device) (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpy(planes)");
  ok();
  return QMM_OK;
}

void qmm_release_weights(qmm_weights* w) {
  if (w == nullptr) return;
  int prev = -1;
  if (hipGetDevice(&prev) == hipSuccess && prev != w->device) (void)hipSetDevice(w->device);
  (void)hipFree(w->alloc);
  if (prev >= 0 && prev != w->device) (void)hipSetDevice(prev);
  g_held -= w->plane_bytes;
  delete w;
}

int qmm_quantize_activations(const float* x, int64_t n_tok, int64_t id, void* qact,
                             size_t qact_bytes, void* stream) {
  if (int rc = check_tokens(n_tok)) return rc;
  if (int rc = check_id(id)) return rc;
  if (n_tok == 0) {  // empty batch: no bytes to write, pointers are not used
    if (qact_bytes != 0) return fail(QMM_EINVAL, "qact_bytes %zu != 0 for n_tok = 0", qact_bytes);
    ok();
    return QMM_OK;
  }
  if (x == nullptr || qact == nullptr) return fail(QMM_EINVAL, "x or qact is NULL");
  if (!aligned(x, 16) || !aligned(qact, 16)) return fail(QMM_EINVAL, "x and qact must be 16-byte aligned");
  const size_t need = qmm_qact_bytes(n_tok, id);
  if (qact_bytes != need)
    return fail(QMM_EINVAL, "qact_bytes %zu != qmm_qact_bytes(%lld, %lld) = %zu", qact_bytes,
                (long long)n_tok, (long long)id, need);
  hipError_t e = qmm::launch_quantize(x, n_tok, token_pad(n_tok), id, (uint8_t*)qact,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "quantize launch");
  ok();
  return QMM_OK;
}

}  // extern "C"

namespace {

// Validation and launch plan shared by qmm_mmq and qmm_mmq_noalloc.  Returns
// QMM_OK with *launch false for an empty batch (nothing to launch).
int prepare_mmq(const qmm_weights* w, const void* qact, size_t qact_bytes, int64_t n_tok, const float* out,
                qmm::MmqPlan* plan, int* device, int* num_cus, bool* launch) {
  *launch = false;
  if (w == nullptr) return fail(QMM_EINVAL, "NULL weights handle");
  if (int rc = check_tokens(n_tok)) return rc;
  if (n_tok == 0) {  // empty batch: an empty output, nothing launched
    if (qact_bytes != 0) return fail(QMM_ESHAPE, "qact_bytes %zu != 0 for n_tok = 0", qact_bytes);
    return QMM_OK;
  }
  if (qact == nullptr || out == nullptr) return fail(QMM_EINVAL, "qact or out is NULL");
  if (!aligned(qact, 16)) return fail(QMM_EINVAL, "qact must be 16-byte aligned");
  if (!aligned(out, 4)) return fail(QMM_EINVAL, "out must be 4-byte aligned");
  const size_t need = qmm_qact_bytes(n_tok, w->p.id);
  if (qact_bytes != need)
    return fail(QMM_ESHAPE, "qact_bytes %zu does not match n_tok=%lld and the handle's id=%lld (%zu)",
                qact_bytes, (long long)n_tok, (long long)w->p.id, need);
  hipError_t e = hipGetDevice(device);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (*device != w->device)
    return fail(QMM_EINVAL, "handle belongs to device %d but device %d is current", w->device, *device);
  e = hipDeviceGetAttribute(num_cus, hipDeviceAttributeMultiprocessorCount, *device);
  if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(multiprocessor count)");
  *plan = qmm::plan_mmq(w->p, n_tok, *num_cus);
  if (int rc = check_launch(*plan, n_tok, w->p.od, *num_cus)) return rc;
  *launch = true;
  return QMM_OK;
}

}  // namespace

extern "C" {

int qmm_mmq(const qmm_weights* w, const void* qact, size_t qact_bytes, int64_t n_tok, float* out,
            void* stream) {
  qmm::MmqPlan plan{};
  int device = -1, num_cus = 0;
  bool launch = false;
  if (int rc = prepare_mmq(w, qact, qact_bytes, n_tok, out, &plan, &device, &num_cus, &launch)) return rc;
  if (!launch) {
    ok();
    return QMM_OK;
  }
  const hipStream_t s = (hipStream_t)stream;
  void* scratch = nullptr;
  if (plan.scratch_bytes > 0) {
    const size_t max_bytes = qmm::mmq_scratch_max_bytes(num_cus);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (const Scratch& sc : g_scratch)
      if (sc.device == device && sc.stream == s) scratch = sc.ptr;
    if (scratch == nullptr) {
      hipError_t e = hipMalloc(&scratch, max_bytes);
      if (e != hipSuccess) {
        (void)hipGetLastError();  // leave no sticky error for the caller's next HIP call
        return e == hipErrorOutOfMemory
                   ? fail(QMM_ENOMEM, "hipMalloc(%zu) for the tail partials failed", max_bytes)
                   : fail_hip(e, "hipMalloc(tail partials)");
      }
      g_scratch.push_back({device, s, scratch, max_bytes});
    }
  }
  hipError_t e = qmm::launch_mmq(w->p, plan, (const uint8_t*)qact, n_tok, token_pad(n_tok), out,
                                 (float*)scratch, s);
  if (e != hipSuccess) return fail_hip(e, "mmq launch");
  ok();
  return QMM_OK;
}

int qmm_stream_release(void* stream, size_t* freed_bytes) {
  const hipStream_t s = (hipStream_t)stream;
  if (freed_bytes != nullptr) *freed_bytes = 0;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  bool synced = false;
  int cur = -1;
  for (size_t i = 0; i < g_scratch.size();) {
    if (g_scratch[i].stream != s) {
      ++i;
      continue;
    }
    // ---- first HIP call below this line (none when the stream holds nothing) ----
    hipError_t e;
    if (!synced) {  // the stream's MMQs may still read the partials
      if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
      if ((e = hipGetDevice(&cur)) != hipSuccess) return fail_hip(e, "hipGetDevice");
      synced = true;
    }
    if ((e = hipSetDevice(g_scratch[i].device)) != hipSuccess) return fail_hip(e, "hipSetDevice");
    e = hipFree(g_scratch[i].ptr);
    const hipError_t e2 = hipSetDevice(cur);
    if (e != hipSuccess) return fail_hip(e, "hipFree(tail partials)");
    if (e2 != hipSuccess) return fail_hip(e2, "hipSetDevice(restore)");
    if (freed_bytes != nullptr) *freed_bytes += g_scratch[i].bytes;
    g_scratch.erase(g_scratch.begin() + (ptrdiff_t)i);
  }
  ok();
  return QMM_OK;
}

int qmm_mmq_noalloc(const qmm_weights* w, const void* qact, size_t qact_bytes, int64_t n_tok, float* out,
                    void* stream) {
  qmm::MmqPlan plan{};
  int device = -1, num_cus = 0;
  bool launch = false;
  if (int rc = prepare_mmq(w, qact, qact_bytes, n_tok, out, &plan, &device, &num_cus, &launch)) return rc;
  if (!launch) {
    ok();
    return QMM_OK;
  }
  if (plan.scratch_bytes > qmm::kStaticScratchBytes)
    return fail(QMM_EINVAL, "this launch needs %zu bytes of tail scratch; the static scratch holds %zu",
                plan.scratch_bytes, qmm::kStaticScratchBytes);
  float* part = nullptr;
  if (plan.scratch_bytes > 0) {
    hipError_t e = qmm::static_scratch(device, &part);
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(static tail scratch)");
  }
  hipError_t e = qmm::launch_mmq(w->p, plan, (const uint8_t*)qact, n_tok, token_pad(n_tok), out, part,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "mmq launch");
  ok();
  return QMM_OK;
}

int qmm_mmq_plan(int type, int64_t od, int64_t id, int64_t n_tok, int num_cus, qmm_plan* out) {
  if (out == nullptr) return fail(QMM_EINVAL, "out is NULL");
  std::memset(out, 0, sizeof *out);
  if (int rc = check_type(type)) return rc;
  if (int rc = check_od(od)) return rc;
  if (int rc = check_id(id)) return rc;
  if (int rc = check_tokens(n_tok)) return rc;
  if (num_cus < 1 || num_cus > QMM_MAX_CUS)
    return fail(QMM_EINVAL, "num_cus must be in [1, %d], got %d", QMM_MAX_CUS, num_cus);
  out->nsb = (int32_t)(id / 256);
  if (n_tok == 0) {  // an empty batch launches nothing
    ok();
    return QMM_OK;
  }
  const qmm::MmqPlan plan = qmm::plan_mmq(plane_shape(type, od, id), n_tok, num_cus);
  if (int rc = check_launch(plan, n_tok, od, num_cus)) return rc;
  out->work_groups = plan.work_groups;
  out->scratch_bytes = plan.scratch_bytes;
  out->threads = plan.threads;
  out->many = plan.many ? 1 : 0;
  out->tile_rows = plan.tile_rows;
  out->tile_tokens = plan.tile_tokens;
  out->k_groups = plan.k_groups;
  out->per_cu = plan.per_cu;
  out->row_tiles = plan.row_tiles;
  out->tok_tiles = plan.tok_tiles;
  out->dp_row_tiles = plan.dp_row_tiles;
  out->n_tail = plan.n_tail;
  out->split = plan.split;
  ok();
  return QMM_OK;
}

int qmm_mmq_plan_work(const qmm_plan* plan, int64_t wg, int32_t* row_tile, int32_t* tok_tile, int32_t* sb_begin,
                      int32_t* sb_end) {
  if (plan == nullptr || row_tile == nullptr || tok_tile == nullptr || sb_begin == nullptr || sb_end == nullptr)
    return fail(QMM_EINVAL, "plan or an output pointer is NULL");
  const qmm_plan& q = *plan;
  const bool consistent = q.nsb >= 1 && q.tok_tiles >= 1 && q.dp_row_tiles >= 0 && q.n_tail >= 0 &&
                          q.split >= 1 && (q.n_tail > 0) == (q.split > 1) && q.split <= q.nsb &&
                          q.n_tail % q.tok_tiles == 0 && q.dp_row_tiles + q.n_tail / q.tok_tiles == q.row_tiles &&
                          q.work_groups == (int64_t)q.dp_row_tiles * q.tok_tiles + (int64_t)q.n_tail * q.split &&
                          q.work_groups < ((int64_t)1 << 31);
  if (!consistent) return fail(QMM_EINVAL, "plan is not one qmm_mmq_plan wrote");
  if (wg < 0 || wg >= q.work_groups)
    return fail(QMM_EINVAL, "work-group %lld outside the launch's %lld", (long long)wg, (long long)q.work_groups);
  qmm::MmqPlan p{};
  p.row_tiles = q.row_tiles;
  p.tok_tiles = q.tok_tiles;
  p.dp_row_tiles = q.dp_row_tiles;
  p.n_tail = q.n_tail;
  p.split = q.split;
  int rt = 0, tt = 0, s0 = 0, s1 = 0;
  qmm::plan_work(p, q.nsb, wg, &rt, &tt, &s0, &s1);
  *row_tile = rt;
  *tok_tile = tt;
  *sb_begin = s0;
  *sb_end = s1;
  ok();
  return QMM_OK;
}

}  // extern "C"
