// C ABI of the rotattn library: argument validation, buffer and workspace
// sizing, and the launch sequence of each call. No device memory is
// allocated here; every scratch buffer is carved out of the caller's
// workspace.
#include "../../include/rotattn.h"
#include "common.h"

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cmath>
#include <cstring>
#include <mutex>

using namespace rotattn;

// Scratch of the allocation-free entry point (rotattn_quantize_qk_static):
// one copy per device, held until the process ends. It holds the RoPE tables
// of one call; every call on a device overwrites it.
constexpr size_t kScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Derived {
  KProblem kp;
  int64_t Lp, NB, Dp;
};

int derive(const rotattn_problem* p, Derived* d) {
  if (p == nullptr) return ROTATTN_EINVAL;
  if (p->B < 1 || p->H < 1 || p->L < 0 || p->text_prefix < 0) return ROTATTN_EINVAL;
  if (p->grid_t < 0 || p->grid_h < 0 || p->grid_w < 0) return ROTATTN_EINVAL;
  if (p->D != 64 && p->D != 128) return ROTATTN_EUNSUPPORTED;
  if (p->rotation != ROTATTN_ROT_FULL && p->rotation != ROTATTN_ROT_GROUP64 && p->rotation != ROTATTN_ROT_PAIR)
    return ROTATTN_EINVAL;
  const int64_t video = (int64_t)p->grid_t * p->grid_h * p->grid_w;
  if ((int64_t)p->text_prefix + video != (int64_t)p->L) return ROTATTN_EINVAL;
  if (p->L > (1 << 30)) return ROTATTN_EUNSUPPORTED;
  // launch limits: a dispatch counts work-items in 32 bits per grid dimension,
  // and the per-(head, block) launches put B*H*NB workgroups of 256 on x
  if (p->H > 65535 || 2 * (int64_t)p->B > 65535) return ROTATTN_EUNSUPPORTED;
  if ((int64_t)p->B * p->H * (((int64_t)p->L + kBlock - 1) / kBlock) * 256 >= (int64_t(1) << 32))
    return ROTATTN_EUNSUPPORTED;
  int sum = 0;
  for (int a = 0; a < 3; ++a) {
    if (p->rope_split[a] < 0) return ROTATTN_EINVAL;
    sum += p->rope_split[a];
  }
  if (sum != p->D) return ROTATTN_EINVAL;
  if (p->rotation == ROTATTN_ROT_GROUP64)
    for (int a = 0; a < 3; ++a)
      if (p->rope_split[a] > 64) return ROTATTN_EUNSUPPORTED;
  if (!(p->rope_base > 0.0) || !std::isfinite(p->rope_base)) return ROTATTN_EINVAL;
  if (std::isnan(p->block_err_tau)) return ROTATTN_EINVAL;
  if (p->stride_l < p->D || p->stride_h < 0 || p->stride_b < 0) return ROTATTN_EINVAL;
  if ((p->stride_l * 2) % 16 != 0 || (p->stride_h * 2) % 16 != 0 || (p->stride_b * 2) % 16 != 0)
    return ROTATTN_EALIGN;

  KProblem& k = d->kp;
  std::memset(&k, 0, sizeof(k));
  k.B = p->B; k.H = p->H; k.L = p->L; k.D = p->D;
  k.Dp = (p->rotation == ROTATTN_ROT_GROUP64) ? 192 : p->D;
  k.NB = (p->L + kBlock - 1) / kBlock;
  k.Lp = k.NB * kBlock;
  k.T = p->grid_t; k.Hh = p->grid_h; k.W = p->grid_w; k.prefix = p->text_prefix;
  // RoPE tables: cos and sin of every (axis, position, pair), counted in
  // 64 bits; the kernels index them with 32-bit offsets
  int off = 0;
  int64_t toff = 0;
  const int npos[3] = {p->grid_t, p->grid_h, p->grid_w};
  for (int a = 0; a < 3; ++a) {
    k.split[a] = p->rope_split[a];
    k.off[a] = off;
    off += p->rope_split[a];
    k.npair[a] = p->rope_split[a] / 2;
    k.tab_off[a] = (int)toff;
    toff += 2 * (int64_t)npos[a] * k.npair[a];
    if (toff > (int64_t)INT32_MAX) return ROTATTN_EUNSUPPORTED;
  }
  k.tab_floats = (int)toff;
  k.rotation = p->rotation;
  // the mergeable rotation: every RoPE pair turned by pi/4 (folded into RoPE)
  k.pair_phase = (p->rotation == ROTATTN_ROT_PAIR) ? 3.14159265358979323846 / 4.0 : 0.0;
  k.pair_c = (float)std::cos(k.pair_phase);
  k.pair_s = (float)std::sin(k.pair_phase);
  k.sb = p->stride_b; k.sh = p->stride_h; k.sl = p->stride_l;
  k.tau = p->block_err_tau;
  k.base = p->rope_base;
  d->Lp = k.Lp; d->NB = k.NB; d->Dp = k.Dp;
  return ROTATTN_OK;
}

// Workspace carve-up of every call. Offsets are 256-byte aligned.
struct Layout {
  size_t tab = 0, absmax = 0, vcodes = 0, vscale = 0, vcolsum = 0, po = 0, pm = 0, pl = 0, qr = 0, kr = 0, img = 0,
         vt = 0;
  size_t total = 0;
};

bool routes(const rotattn_problem* p) { return std::isfinite(p->block_err_tau); }

Layout layout(const rotattn_problem* p, const Derived& d, int call) {
  Layout L;
  size_t o = 0;
  const int64_t BH = (int64_t)p->B * p->H;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
  const size_t tab_bytes = (size_t)d.kp.tab_floats * sizeof(float) + 16;
  const size_t vcodes_b = (size_t)BH * d.NB * p->D * 32;
  const size_t vscale_b = (size_t)BH * p->D * sizeof(float);
  const size_t vcolsum_b = (size_t)BH * d.NB * p->D * sizeof(int32_t);
  const size_t absmax_b = (size_t)BH * p->D * sizeof(uint32_t);
  const size_t po_b = (size_t)BH * d.Lp * p->D * sizeof(float);
  const size_t pm_b = (size_t)BH * d.Lp * sizeof(float);
  const size_t rope_b = (size_t)BH * p->L * p->D * 2;
  const size_t img_b = (size_t)BH * d.NB * kv_image_bytes((int)d.Dp, p->D);
  const size_t vt_b = (size_t)BH * d.NB * f16_vt_bytes(p->D);
  // the V^T blocks only when the FP16 path can run: block routing on, or a head mask passed
  const bool fp16 = routes(p) || call == ROTATTN_CALL_ATTENTION_HEAD_FALLBACK ||
                    call == ROTATTN_CALL_FORWARD_HEAD_FALLBACK;
  switch (call) {
    case ROTATTN_CALL_QUANTIZE_QK:
      L.tab = take(tab_bytes);
      break;
    case ROTATTN_CALL_QUANTIZE_V:
      L.absmax = take(absmax_b);
      break;
    case ROTATTN_CALL_ATTENTION:
    case ROTATTN_CALL_ATTENTION_HEAD_FALLBACK:
      L.img = take(img_b);
      if (fp16) L.vt = take(vt_b);
      if (routes(p)) { L.po = take(po_b); L.pm = take(pm_b); L.pl = take(pm_b); }
      break;
    case ROTATTN_CALL_FORWARD:
    case ROTATTN_CALL_FORWARD_HEAD_FALLBACK:
      L.vcodes = take(vcodes_b); L.vscale = take(vscale_b); L.vcolsum = take(vcolsum_b);
      L.absmax = take(absmax_b);
      L.img = take(img_b);
      if (fp16) L.vt = take(vt_b);
      if (routes(p)) { L.po = take(po_b); L.pm = take(pm_b); L.pl = take(pm_b); }
      break;
    case ROTATTN_CALL_FP16_FORWARD:
      L.tab = take(tab_bytes); L.qr = take(rope_b); L.kr = take(rope_b); L.vt = take(vt_b);
      break;
    case ROTATTN_CALL_DEBUG_DUMP:
    case ROTATTN_CALL_SPARSE_ATTENTION:
      L.img = take(img_b);
      break;
    case ROTATTN_CALL_BLOCK_MASK:   // no scratch
      break;
    default:
      break;
  }
  L.total = o;
  return L;
}

int check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (L.total == 0) return ROTATTN_OK;
  if (ws == nullptr || ws_bytes < L.total) return ROTATTN_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return ROTATTN_EALIGN;
  return ROTATTN_OK;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int launched(hipError_t e) { return e == hipSuccess ? ROTATTN_OK : ROTATTN_ELAUNCH; }

int check_qk(const rotattn_qk_buffers* qk) {
  if (qk == nullptr || !qk->q_codes || !qk->k_codes || !qk->q_scale || !qk->k_scale || !qk->q_flag ||
      !qk->k_flag || !qk->head_kflag)
    return ROTATTN_EINVAL;
  if (!aligned16(qk->q_codes) || !aligned16(qk->k_codes)) return ROTATTN_EALIGN;
  if ((qk->q_rope && !aligned16(qk->q_rope)) || (qk->k_rope && !aligned16(qk->k_rope))) return ROTATTN_EALIGN;
  if (((uintptr_t)qk->q_scale & 3) || ((uintptr_t)qk->k_scale & 3) || ((uintptr_t)qk->head_kflag & 3))
    return ROTATTN_EALIGN;
  return ROTATTN_OK;
}

int check_v(const rotattn_v_buffers* vq) {
  if (vq == nullptr || !vq->v_codes || !vq->v_scale || !vq->v_colsum) return ROTATTN_EINVAL;
  if (!aligned16(vq->v_codes) || ((uintptr_t)vq->v_scale & 3) || ((uintptr_t)vq->v_colsum & 3))
    return ROTATTN_EALIGN;
  return ROTATTN_OK;
}

// One side stream (default priority, non-blocking) and a fork and a join
// event per device, created on the first call that needs them and kept until
// the process ends; the mutex keeps the record/wait sequences of concurrent
// calls on one device from interleaving.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream* g_side[kMaxSideDevices] = {};

int side_stream(hipStream_t s, SideStream** out) {
  int dev = -1;
  if (s != nullptr) {
    if (hipStreamGetDevice(s, &dev) != hipSuccess) return ROTATTN_EINVAL;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return ROTATTN_ELAUNCH;
  }
  if (dev < 0 || dev >= kMaxSideDevices) return ROTATTN_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_side_mu);
  if (g_side[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ROTATTN_ELAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ROTATTN_ELAUNCH;
    SideStream* ss = new SideStream();
    const bool ok = hipStreamCreateWithFlags(&ss->stream, hipStreamNonBlocking) == hipSuccess &&
                    hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) == hipSuccess &&
                    hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) == hipSuccess;
    if (!ok) {   // release what was created
      if (ss->join != nullptr) (void)hipEventDestroy(ss->join);
      if (ss->fork != nullptr) (void)hipEventDestroy(ss->fork);
      if (ss->stream != nullptr) (void)hipStreamDestroy(ss->stream);
      delete ss;
    }
    const bool restored = cur == dev || hipSetDevice(cur) == hipSuccess;
    if (!ok || !restored) {
      if (ok) g_side[dev] = ss;   // created: keep it for the next call
      return ROTATTN_ELAUNCH;
    }
    g_side[dev] = ss;
  }
  *out = g_side[dev];
  return ROTATTN_OK;
}

int attention_impl(const rotattn_problem* p, const Derived& d, const rotattn_qk_buffers* qk,
                   const rotattn_v_buffers* vq, const void* v, const uint8_t* head_fallback, void* out,
                   void* ws, const Layout& L, hipStream_t s) {
  const bool route = routes(p);
  const bool fp16_needed = route || head_fallback != nullptr;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q_codes = qk->q_codes; a.k_codes = qk->k_codes;
  a.q_scale = qk->q_scale; a.k_scale = qk->k_scale;
  a.q_flag = qk->q_flag; a.k_flag = qk->k_flag; a.head_kflag = qk->head_kflag;
  a.head_mask = head_fallback;
  a.v_codes = vq->v_codes; a.v_scale = vq->v_scale;
  a.q_rope = static_cast<const __half*>(qk->q_rope);
  a.k_rope = static_cast<const __half*>(qk->k_rope);
  a.v = static_cast<const __half*>(v);
  a.out = static_cast<__half*>(out);
  a.route = route;
  if (route) { a.part_o = at<float>(ws, L.po); a.part_m = at<float>(ws, L.pm); a.part_l = at<float>(ws, L.pl); }
  uint8_t* img = at<uint8_t>(ws, L.img);
  a.kv_image = img;
  int rc = launched(launch_kv_image(d.kp, a, img, s));
  if (rc != ROTATTN_OK) return rc;
  if (fp16_needed) {   // V^T blocks of the FP16 tiles, which both kernels read
    uint8_t* vt = at<uint8_t>(ws, L.vt);
    a.f16_vt = vt;
    if ((rc = launched(launch_fp16_vt(d.kp, a.v, vt, s))) != ROTATTN_OK) return rc;
  }
  if (!fp16_needed) return launched(launch_int4_attention(d.kp, a, false, s));
  // Rows that run whole on FP16 do not depend on the INT4 rows: they go to the
  // device's side stream, forked from and joined back into the caller's
  // stream, so that the two kernels share the machine. The INT4 rows (rows
  // that mix both paths: their FP16 tiles too, or, in heads with many flagged
  // K blocks, their INT4 partials), then the merges of those partials, stay
  // on the caller's stream.
  SideStream* ss = nullptr;
  if ((rc = side_stream(s, &ss)) != ROTATTN_OK) return rc;
  std::lock_guard<std::mutex> lock(ss->mu);
  if (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->stream, ss->fork, 0) != hipSuccess)
    return ROTATTN_ELAUNCH;
  if ((rc = launched(launch_fp16_attention(d.kp, a, kFp16FullOnly, ss->stream))) != ROTATTN_OK) return rc;
  if ((rc = launched(launch_int4_attention(d.kp, a, false, s))) != ROTATTN_OK) return rc;
  if (route && (rc = launched(launch_fp16_attention(d.kp, a, kFp16MergeOnly, s))) != ROTATTN_OK) return rc;
  if (hipEventRecord(ss->join, ss->stream) != hipSuccess || hipStreamWaitEvent(s, ss->join, 0) != hipSuccess)
    return ROTATTN_ELAUNCH;
  return ROTATTN_OK;
}

int check_attention_args(const rotattn_problem* p, const rotattn_qk_buffers* qk, const void* v,
                         const uint8_t* head_fallback, const void* out) {
  if (out == nullptr) return ROTATTN_EINVAL;
  if (!aligned16(out)) return ROTATTN_EALIGN;
  const bool fp16_needed = routes(p) || head_fallback != nullptr;
  if (fp16_needed) {
    if (v == nullptr || qk->q_rope == nullptr || qk->k_rope == nullptr) return ROTATTN_EINVAL;
    if (!aligned16(v)) return ROTATTN_EALIGN;
  }
  return ROTATTN_OK;
}

int check_quantize_qk(const void* q, const void* k, const rotattn_qk_buffers* out) {
  if (q == nullptr || k == nullptr) return ROTATTN_EINVAL;
  const int rc = check_qk(out);
  if (rc != ROTATTN_OK) return rc;
  if (!aligned16(q) || !aligned16(k)) return ROTATTN_EALIGN;
  return ROTATTN_OK;
}

// RoPE tables into `tab` (also clears head_kflag), then the Q/K prologue.
int quantize_qk_impl(const rotattn_problem* p, const Derived& d, const void* q, const void* k,
                     const rotattn_qk_buffers* out, float* tab, hipStream_t s) {
  int rc = launched(launch_rope_tables(d.kp, tab, out->head_kflag, p->B * p->H, d.kp.pair_phase, s));
  if (rc != ROTATTN_OK) return rc;
  QKOut o;
  o.q_codes = out->q_codes; o.k_codes = out->k_codes;
  o.q_scale = out->q_scale; o.k_scale = out->k_scale;
  o.q_flag = out->q_flag; o.k_flag = out->k_flag;
  o.head_kflag = out->head_kflag;
  o.q_rope = static_cast<__half*>(out->q_rope);
  o.k_rope = static_cast<__half*>(out->k_rope);
  o.q_bsum = out->q_bsum;
  o.k_bsum = out->k_bsum;
  return launched(launch_qk_prologue(d.kp, static_cast<const __half*>(q), static_cast<const __half*>(k), tab, o, s));
}

// Device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept: in host code the array's name
// is only a host-side handle, never a device address. The stream must belong
// to the current device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int scratch_on_stream_device(hipStream_t s, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ROTATTN_ELAUNCH;
  if (s != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return ROTATTN_EINVAL;
    if (sdev != dev) return ROTATTN_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return ROTATTN_ELAUNCH;
    g_scratch_dev[dev] = addr;
  }
  *ptr = g_scratch_dev[dev];
  return ROTATTN_OK;
}

}  // namespace

extern "C" {

int rotattn_version(void) { return ROTATTN_VERSION; }

const char* rotattn_strerror(int code) {
  switch (code) {
    case ROTATTN_OK: return "success";
    case ROTATTN_EINVAL: return "invalid argument (null pointer, size, split, grid or stride)";
    case ROTATTN_EUNSUPPORTED:
      return "unsupported problem (head dim must be 64 or 128; RoPE groups <= 64 for ROT_GROUP64; L <= 2^30, "
             "H <= 65535, 2B <= 65535, B*H*ceil(L/64) < 2^24, RoPE tables < 2^31 floats)";
    case ROTATTN_EALIGN: return "pointer or row stride not 16-byte aligned (workspace: 256-byte)";
    case ROTATTN_EWORKSPACE: return "workspace missing or too small";
    case ROTATTN_ELAUNCH: return "kernel launch failed";
    case ROTATTN_ESCRATCH:
      return "problem needs more scratch than the static buffer of the allocation-free entry point holds (1 MiB)";
    default: return "unknown error code";
  }
}

int rotattn_get_sizes(const rotattn_problem* p, rotattn_sizes* out) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (out == nullptr) return ROTATTN_EINVAL;
  const int64_t BH = (int64_t)p->B * p->H;
  out->Lp = d.Lp; out->NB = d.NB; out->Dp = d.Dp;
  out->qk_codes_bytes = BH * d.Lp * d.Dp / 2;
  out->qk_scale_bytes = BH * d.NB * 4;
  out->qk_flag_bytes = BH * d.NB;
  out->head_flag_bytes = BH * 4;
  out->rope_bytes = BH * p->L * p->D * 2;
  out->v_codes_bytes = BH * d.NB * p->D * 32;
  out->v_scale_bytes = BH * p->D * 4;
  out->v_colsum_bytes = BH * d.NB * p->D * 4;
  out->bsum_bytes = BH * d.NB * p->D * 4;
  out->mask_rows = (d.NB + 1) / 2;
  out->mask_words = (d.NB + 31) / 32;
  out->mask_bytes = BH * out->mask_rows * out->mask_words * 4;
  out->out_min_elems = (p->L == 0) ? 0
      : (int64_t)(p->B - 1) * p->stride_b + (int64_t)(p->H - 1) * p->stride_h + (int64_t)(p->L - 1) * p->stride_l + p->D;
  return ROTATTN_OK;
}

int rotattn_workspace_bytes(const rotattn_problem* p, int call, size_t* bytes) {
  Derived d;
  const int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (bytes == nullptr || call < 0 || call > ROTATTN_CALL_FORWARD_HEAD_FALLBACK) return ROTATTN_EINVAL;
  *bytes = layout(p, d, call).total;
  return ROTATTN_OK;
}

int rotattn_quantize_qk(const rotattn_problem* p, const void* q, const void* k, const rotattn_qk_buffers* out,
                        void* workspace, size_t workspace_bytes, rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if ((rc = check_quantize_qk(q, k, out)) != ROTATTN_OK) return rc;
  const Layout L = layout(p, d, ROTATTN_CALL_QUANTIZE_QK);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  return quantize_qk_impl(p, d, q, k, out, at<float>(workspace, L.tab), static_cast<hipStream_t>(stream));
}

int rotattn_quantize_qk_static(const rotattn_problem* p, const void* q, const void* k,
                               const rotattn_qk_buffers* out, rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if ((rc = check_quantize_qk(q, k, out)) != ROTATTN_OK) return rc;
  if (layout(p, d, ROTATTN_CALL_QUANTIZE_QK).total > kScratchBytes) return ROTATTN_ESCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* scr = nullptr;
  if ((rc = scratch_on_stream_device(s, &scr)) != ROTATTN_OK) return rc;
  // the tables are written whole by every call before the prologue reads them: nothing to clear
  return quantize_qk_impl(p, d, q, k, out, static_cast<float*>(scr), s);
}

int rotattn_quantize_v(const rotattn_problem* p, const void* v, const rotattn_v_buffers* out, void* workspace,
                       size_t workspace_bytes, rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if (v == nullptr) return ROTATTN_EINVAL;
  if ((rc = check_v(out)) != ROTATTN_OK) return rc;
  if (!aligned16(v)) return ROTATTN_EALIGN;
  const Layout L = layout(p, d, ROTATTN_CALL_QUANTIZE_V);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;
  VOut o{out->v_codes, out->v_scale, out->v_colsum};
  return launched(launch_vquant(d.kp, static_cast<const __half*>(v), at<uint32_t>(workspace, L.absmax), o,
                                static_cast<hipStream_t>(stream)));
}

int rotattn_attention(const rotattn_problem* p, const rotattn_qk_buffers* qk, const rotattn_v_buffers* vq,
                      const void* v, const uint8_t* head_fallback, void* out, void* workspace,
                      size_t workspace_bytes, rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if ((rc = check_qk(qk)) != ROTATTN_OK) return rc;
  if ((rc = check_v(vq)) != ROTATTN_OK) return rc;
  if ((rc = check_attention_args(p, qk, v, head_fallback, out)) != ROTATTN_OK) return rc;
  const Layout L = layout(p, d, head_fallback ? ROTATTN_CALL_ATTENTION_HEAD_FALLBACK : ROTATTN_CALL_ATTENTION);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;
  return attention_impl(p, d, qk, vq, v, head_fallback, out, workspace, L, static_cast<hipStream_t>(stream));
}

int rotattn_forward(const rotattn_problem* p, const rotattn_qk_buffers* qk, const void* v,
                    const uint8_t* head_fallback, void* out, void* workspace, size_t workspace_bytes,
                    rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if ((rc = check_qk(qk)) != ROTATTN_OK) return rc;
  if (v == nullptr) return ROTATTN_EINVAL;
  if (!aligned16(v)) return ROTATTN_EALIGN;
  if ((rc = check_attention_args(p, qk, v, head_fallback, out)) != ROTATTN_OK) return rc;
  const Layout L = layout(p, d, head_fallback ? ROTATTN_CALL_FORWARD_HEAD_FALLBACK : ROTATTN_CALL_FORWARD);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  VOut o{at<uint8_t>(workspace, L.vcodes), at<float>(workspace, L.vscale), at<int32_t>(workspace, L.vcolsum)};
  rc = launched(launch_vquant(d.kp, static_cast<const __half*>(v), at<uint32_t>(workspace, L.absmax), o, s));
  if (rc != ROTATTN_OK) return rc;
  rotattn_v_buffers vq{o.v_codes, o.v_scale, o.v_colsum};
  return attention_impl(p, d, qk, &vq, v, head_fallback, out, workspace, L, s);
}

int rotattn_fp16_forward(const rotattn_problem* p, const void* q, const void* k, const void* v, void* out,
                         void* workspace, size_t workspace_bytes, rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return ROTATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ROTATTN_EALIGN;
  const Layout L = layout(p, d, ROTATTN_CALL_FP16_FORWARD);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* tab = at<float>(workspace, L.tab);
  __half* qr = at<__half>(workspace, L.qr);
  __half* kr = at<__half>(workspace, L.kr);
  if ((rc = launched(launch_rope_tables(d.kp, tab, nullptr, 0, 0.0, s))) != ROTATTN_OK) return rc;   // plain RoPE
  if ((rc = launched(launch_rope_copy(d.kp, static_cast<const __half*>(q), tab, qr, s))) != ROTATTN_OK) return rc;
  if ((rc = launched(launch_rope_copy(d.kp, static_cast<const __half*>(k), tab, kr, s))) != ROTATTN_OK) return rc;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q_rope = qr; a.k_rope = kr;
  a.v = static_cast<const __half*>(v);
  a.out = static_cast<__half*>(out);
  a.route = false;
  uint8_t* vt = at<uint8_t>(workspace, L.vt);
  a.f16_vt = vt;
  if ((rc = launched(launch_fp16_vt(d.kp, a.v, vt, s))) != ROTATTN_OK) return rc;
  return launched(launch_fp16_attention(d.kp, a, kFp16WholeCall, s));
}

int rotattn_debug_dump(const rotattn_problem* p, const rotattn_qk_buffers* qk, const rotattn_v_buffers* vq,
                       const uint8_t* head_fallback, const uint32_t* block_mask, const int32_t* units,
                       int32_t n_units, int32_t* acc_qk,
                       int8_t* p_codes, int32_t* acc_pv, float* m_hist, float* p15, void* workspace,
                       size_t workspace_bytes, rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if ((rc = check_qk(qk)) != ROTATTN_OK) return rc;
  if ((rc = check_v(vq)) != ROTATTN_OK) return rc;
  if (n_units < 0 || (n_units > 0 && (!units || !acc_qk || !p_codes || !acc_pv || !m_hist))) return ROTATTN_EINVAL;
  if (block_mask != nullptr) {
    if (((uintptr_t)block_mask & 3) != 0) return ROTATTN_EALIGN;
    if (routes(p) || head_fallback != nullptr) return ROTATTN_EINVAL;
  }
  const Layout L = layout(p, d, ROTATTN_CALL_DEBUG_DUMP);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  if (n_units == 0 || p->L == 0) return ROTATTN_OK;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q_codes = qk->q_codes; a.k_codes = qk->k_codes;
  a.q_scale = qk->q_scale; a.k_scale = qk->k_scale;
  a.q_flag = qk->q_flag; a.k_flag = qk->k_flag; a.head_kflag = qk->head_kflag;
  a.head_mask = head_fallback;
  a.v_codes = vq->v_codes; a.v_scale = vq->v_scale;
  a.route = routes(p);
  a.units = units; a.n_units = n_units;
  a.d_acc = acc_qk; a.d_pq = p_codes; a.d_pv = acc_pv; a.d_m = m_hist; a.d_p15 = p15;
  a.block_mask = block_mask;
  a.mask_words = (int)((d.NB + 31) / 32);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* img = at<uint8_t>(workspace, L.img);
  a.kv_image = img;
  if ((rc = launched(launch_kv_image(d.kp, a, img, s))) != ROTATTN_OK) return rc;
  return launched(launch_int4_attention(d.kp, a, true, s));
}

int rotattn_block_mask(const rotattn_problem* p, const rotattn_qk_buffers* qk, int32_t topn, uint32_t* mask,
                       void* workspace, size_t workspace_bytes, rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if (qk == nullptr || qk->q_bsum == nullptr || qk->k_bsum == nullptr || mask == nullptr || topn < 1)
    return ROTATTN_EINVAL;
  if (d.NB > kMaxMaskBlocks || (int64_t)p->B * p->H > 65535) return ROTATTN_EUNSUPPORTED;
  if (!aligned16(qk->q_bsum) || !aligned16(qk->k_bsum)) return ROTATTN_EALIGN;
  if (((uintptr_t)mask & 3) != 0) return ROTATTN_EALIGN;
  const Layout L = layout(p, d, ROTATTN_CALL_BLOCK_MASK);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  // text prefix + first frame: the tokens that take part in full attention
  const int64_t frame = (p->grid_t > 0) ? (int64_t)p->grid_h * p->grid_w : 0;
  const int64_t sink_end = std::min<int64_t>(p->L, (int64_t)p->text_prefix + frame);
  const int sink_rows = (int)((sink_end + kMaskQBlock - 1) / kMaskQBlock);
  const int sink_cols = (int)((sink_end + kBlock - 1) / kBlock);
  return launched(launch_block_topn(d.kp, qk->q_bsum, qk->k_bsum, topn, sink_rows, sink_cols, mask,
                                    static_cast<hipStream_t>(stream)));
}

int rotattn_sparse_attention(const rotattn_problem* p, const rotattn_qk_buffers* qk, const rotattn_v_buffers* vq,
                             const uint32_t* block_mask, void* out, void* workspace, size_t workspace_bytes,
                             rotattn_stream_t stream) {
  Derived d;
  int rc = derive(p, &d);
  if (rc != ROTATTN_OK) return rc;
  if (p->L == 0) return ROTATTN_OK;   // nothing to do; zero-size buffers may be null
  if ((rc = check_qk(qk)) != ROTATTN_OK) return rc;
  if ((rc = check_v(vq)) != ROTATTN_OK) return rc;
  if (block_mask == nullptr || out == nullptr || routes(p)) return ROTATTN_EINVAL;
  if (((uintptr_t)block_mask & 3) != 0 || !aligned16(out)) return ROTATTN_EALIGN;
  const Layout L = layout(p, d, ROTATTN_CALL_SPARSE_ATTENTION);
  if ((rc = check_ws(L, workspace, workspace_bytes)) != ROTATTN_OK) return rc;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q_codes = qk->q_codes; a.k_codes = qk->k_codes;
  a.q_scale = qk->q_scale; a.k_scale = qk->k_scale;
  a.q_flag = qk->q_flag; a.k_flag = qk->k_flag; a.head_kflag = qk->head_kflag;
  a.v_codes = vq->v_codes; a.v_scale = vq->v_scale;
  a.out = static_cast<__half*>(out);
  a.route = false;
  a.block_mask = block_mask;
  a.mask_words = (int)((d.NB + 31) / 32);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* img = at<uint8_t>(workspace, L.img);
  a.kv_image = img;
  if ((rc = launched(launch_kv_image(d.kp, a, img, s))) != ROTATTN_OK) return rc;
  return launched(launch_int4_attention(d.kp, a, false, s));
}

}  // extern "C"
