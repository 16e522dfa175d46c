// C ABI entry points: plan upload/destroy, argument validation, kernel
// launches of the forward and backward, and the optional kernel timing.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "plan.h"

using ba::fail;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2i(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// ---- kernel timing -------------------------------------------------------
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> ev0, ev1;
  std::vector<std::string> names;
  size_t used = 0;
};
Profiler &prof() {
  static Profiler *p = new Profiler();  // never destroyed: safe at process exit
  return *p;
}

template <class F>
hipError_t timed(const char *name, hipStream_t s, F &&launch) {
  Profiler &P = prof();
  size_t slot = SIZE_MAX;
  {
    std::lock_guard<std::mutex> g(P.mu);
    if (P.on && P.used < P.ev0.size()) {
      slot = P.used++;
      P.names[slot] = name;
    }
  }
  if (slot != SIZE_MAX) {
    hipError_t e = hipEventRecord(P.ev0[slot], s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (e != hipSuccess) return e;
  if (slot != SIZE_MAX) return hipEventRecord(P.ev1[slot], s);
  return hipSuccess;
}

ba_status hip_fail(const char *what, hipError_t e) {
  return fail(BA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

ba_status check_plan(const ba_plan *p) {
  if (p == nullptr) return fail(BA_E_INVALID, "plan is NULL");
  int uploaded_to = -1;
  {
    std::lock_guard<std::mutex> g(p->dev_mu);
    if (p->dev.block == nullptr)
      return fail(BA_E_INVALID, "plan not uploaded (call ba_plan_upload)");
    uploaded_to = p->dev.device;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(BA_E_HIP, "hipGetDevice failed");
  if (dev != uploaded_to) return fail(BA_E_INVALID, "plan was uploaded to another device");
  return BA_OK;
}

// ---- static scratch of the no-allocation forward ---------------------------
// Device memory of branch_attn_fwd_static: the forward's workspace (the fp32
// main-key partial and its LSE of every branch row) lives in this array
// instead of a caller buffer. Every GPU the library runs on holds its own
// copy for the life of the process. Host code never uses the array's name as
// an address: its device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_ptrs().
constexpr size_t kStaticScratchBytes = size_t(256) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

struct ScratchPtrs {
  std::mutex mu;
  std::vector<void *> ptr;  // per device ordinal; nullptr until looked up
};
ScratchPtrs &scratch_ptrs() {
  static ScratchPtrs *s = new ScratchPtrs();  // never destroyed: safe at process exit
  return *s;
}

// Device address of `scratch` on the current device, looked up on the first
// call for that device.
ba_status scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BA_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  ScratchPtrs &S = scratch_ptrs();
  std::lock_guard<std::mutex> g(S.mu);
  if (S.ptr.size() <= size_t(dev)) S.ptr.resize(size_t(dev) + 1, nullptr);
  if (S.ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(BA_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    S.ptr[dev] = ptr;
  }
  *out = S.ptr[dev];
  return BA_OK;
}

float resolve_scale(float s, int d) { return s > 0.f ? s : 1.0f / std::sqrt(float(d)); }

ba::F32Shape f32_shape(const ba_plan &p, float scale) {
  ba::F32Shape sh{};
  sh.bound_main = p.dev.bound_main;
  sh.bound_branch = p.dev.bound_branch;
  sh.branch_seq = p.dev.branch_seq;
  sh.row_seq = p.dev.row_seq;
  sh.cu_local = p.dev.cu_local;
  sh.chunk = p.dev.chunk;
  sh.seq_len = p.dev.seq_len;
  sh.seq_a0 = p.dev.seq_a0;
  sh.branch_off = p.dev.branch_off;
  sh.anchor_pos = p.dev.anchor_pos;
  sh.n_local = int32_t(p.n_local);
  sh.n_branch = int32_t(p.n_branch);
  sh.n_seqs = p.n_seqs;
  sh.hq = p.hq;
  sh.hkv = p.hkv;
  sh.G = p.G;
  sh.C = p.C;
  sh.r = p.r;
  sh.d = p.d;
  sh.scale = scale;
  sh.scale_log2 = scale * ba::kLog2eHost;
  return sh;
}

}  // namespace

extern "C" ba_status ba_plan_upload(ba_plan *p) {
  try {
    if (p == nullptr) return fail(BA_E_INVALID, "plan is NULL");
    std::lock_guard<std::mutex> guard(p->dev_mu);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    // set-up of this device for the no-allocation forward as well
    void *scr = nullptr;
    ba_status st = scratch_on_current_device(&scr);
    if (st != BA_OK) return st;
    if (p->dev.block != nullptr) {
      if (dev == p->dev.device) return BA_OK;
      return fail(BA_E_INVALID, "plan already uploaded to device " + std::to_string(p->dev.device));
    }
    // one staging buffer, every array at a 256-byte boundary
    std::vector<char> host;
    auto put = [&](const void *src, size_t bytes) -> size_t {
      const size_t off = (host.size() + 255) & ~size_t(255);
      host.resize(off + std::max<size_t>(bytes, 4));
      if (bytes) std::memcpy(host.data() + off, src, bytes);
      return off;
    };
    auto put32 = [&](const std::vector<int32_t> &v) { return put(v.data(), v.size() * 4); };
    const size_t o_bm = put32(p->bound_main), o_bb = put32(p->bound_branch),
                 o_ba = put32(p->b_anchor), o_bo = put32(p->branch_off),
                 o_qt = put(p->qtiles.data(), p->qtiles.size() * sizeof(ba::QTile)),
                 o_kt = put(p->ktiles.data(), p->ktiles.size() * sizeof(ba::KTile)),
                 o_bt = put(p->btiles.data(), p->btiles.size() * sizeof(ba::BTile)),
                 o_rs = put32(p->seq), o_bs = put32(p->branch_seq), o_cl = put32(p->cu_local),
                 o_ch = put32(p->c), o_sl = put32(p->L), o_sa = put32(p->seq_a0),
                 o_ap = put32(p->anchor_pos);
    void *block = nullptr;
    e = hipMalloc(&block, host.size());
    if (e != hipSuccess) return fail(BA_E_OOM, std::string("hipMalloc: ") + hipGetErrorString(e));
    e = hipMemcpy(block, host.data(), host.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(block);
      return hip_fail("hipMemcpy", e);
    }
    char *b = static_cast<char *>(block);
    auto at = [&](size_t off) { return reinterpret_cast<const int32_t *>(b + off); };
    p->dev.device = dev;
    p->dev.block = block;
    p->dev.bound_main = at(o_bm);
    p->dev.bound_branch = at(o_bb);
    p->dev.b_anchor = at(o_ba);
    p->dev.branch_off = at(o_bo);
    p->dev.qtiles = reinterpret_cast<const ba::QTile *>(b + o_qt);
    p->dev.ktiles = reinterpret_cast<const ba::KTile *>(b + o_kt);
    p->dev.btiles = reinterpret_cast<const ba::BTile *>(b + o_bt);
    p->dev.row_seq = at(o_rs);
    p->dev.branch_seq = at(o_bs);
    p->dev.cu_local = at(o_cl);
    p->dev.chunk = at(o_ch);
    p->dev.seq_len = at(o_sl);
    p->dev.seq_a0 = at(o_sa);
    p->dev.anchor_pos = at(o_ap);
    return BA_OK;
  } catch (const std::bad_alloc &) {
    return fail(BA_E_OOM, "host allocation failed while uploading");
  } catch (...) {
    return fail(BA_E_INVALID, "unexpected error while uploading");
  }
}

extern "C" void ba_plan_destroy(ba_plan *p) {
  if (p == nullptr) return;
  if (p->dev.block != nullptr) {
    int cur = -1;
    const bool have = hipGetDevice(&cur) == hipSuccess;
    if (have && cur != p->dev.device) (void)hipSetDevice(p->dev.device);
    (void)hipFree(p->dev.block);
    if (have && cur != p->dev.device) (void)hipSetDevice(cur);
  }
  delete p;
}

namespace {

// The forward with its workspace given explicitly (the caller's buffer, or
// the static scratch); the plan has been checked.
ba_status fwd_impl(const ba_plan *p, const ba_fwd_args *a, void *workspace, size_t workspace_bytes,
                   void *stream);

}  // namespace

extern "C" ba_status branch_attn_fwd(const ba_plan *p, const ba_fwd_args *a, void *stream) {
  try {
    ba_status st = check_plan(p);
    if (st != BA_OK) return st;
    if (a == nullptr) return fail(BA_E_INVALID, "args is NULL");
    return fwd_impl(p, a, a->workspace, a->workspace_bytes, stream);
  } catch (...) {
    return fail(BA_E_INVALID, "unexpected error in branch_attn_fwd");
  }
}

extern "C" ba_status branch_attn_fwd_static(const ba_plan *p, const ba_fwd_args *a, void *stream) {
  try {
    ba_status st = check_plan(p);
    if (st != BA_OK) return st;
    if (p->ws_fwd > kStaticScratchBytes)
      return fail(BA_E_WORKSPACE, "the plan's forward workspace (" + std::to_string(p->ws_fwd) +
                                      " bytes) exceeds the static scratch (" +
                                      std::to_string(kStaticScratchBytes) + " bytes)");
    if (a == nullptr) return fail(BA_E_INVALID, "args is NULL");
    if (a->workspace != nullptr || a->workspace_bytes != 0)
      return fail(BA_E_INVALID, "branch_attn_fwd_static takes no workspace (pass NULL and 0)");
    void *scr = nullptr;
    st = scratch_on_current_device(&scr);
    if (st != BA_OK) return st;
    return fwd_impl(p, a, scr, kStaticScratchBytes, stream);
  } catch (...) {
    return fail(BA_E_INVALID, "unexpected error in branch_attn_fwd_static");
  }
}

namespace {

ba_status fwd_impl(const ba_plan *p, const ba_fwd_args *a, void *workspace, size_t workspace_bytes,
                   void *stream) {
  try {
    if (!a->q || !a->k || !a->v || !a->o || !a->lse)
      return fail(BA_E_INVALID, "q, k, v, o and lse are required");
    const bool has_b = p->n_branch > 0;
    if (has_b && (!a->qb || !a->kb || !a->vb || !a->ob || !a->lseb))
      return fail(BA_E_INVALID, "qb, kb, vb, ob and lseb are required when the plan has branch rows");
    for (const void *ptr : {a->q, a->k, a->v, (const void *)a->o, (const void *)a->lse, a->qb, a->kb,
                            a->vb, (const void *)a->ob, (const void *)a->lseb, (const void *)workspace})
      if (!aligned16(ptr)) return fail(BA_E_INVALID, "every pointer must be 16-byte aligned");
    if (p->ws_fwd > 0 && (workspace == nullptr || workspace_bytes < p->ws_fwd))
      return fail(BA_E_WORKSPACE, "forward workspace needs " + std::to_string(p->ws_fwd) + " bytes");
    if (!(std::isfinite(a->scale))) return fail(BA_E_INVALID, "scale must be finite");
    const float scale = resolve_scale(a->scale, p->d);
    hipStream_t s = static_cast<hipStream_t>(stream);

    float *om = nullptr, *lm = nullptr;
    if (has_b) {
      om = static_cast<float *>(workspace);
      const size_t om_bytes = (size_t(p->n_branch) * p->hq * p->d * 4 + 255) & ~size_t(255);
      lm = reinterpret_cast<float *>(static_cast<char *>(workspace) + om_bytes);
    }
    ba::FwdRingArgs ra{};
    ra.q = a->q;
    ra.qb = a->qb;
    ra.k = a->k;
    ra.v = a->v;
    ra.o = a->o;
    ra.lse = a->lse;
    ra.om = om;
    ra.lm = lm;
    ra.qtiles = p->dev.qtiles;
    ra.bound_main = p->dev.bound_main;
    ra.bound_branch = p->dev.bound_branch;
    ra.n_local = int32_t(p->n_local);
    ra.n_branch = int32_t(p->n_branch);
    ra.hq = p->hq;
    ra.hkv = p->hkv;
    ra.G = p->G;
    ra.log2G = log2i(p->G);
    ra.C = p->C;
    ra.r = p->r;
    ra.d = p->d;
    ra.scale = scale;
    ra.scale_log2 = scale * ba::kLog2eHost;
    ra.runs = ba::uses_run_walk(*p) ? 1 : 0;
    hipError_t e;
    if (p->dtype == BA_BF16) {
      e = timed("fwd_ring", s, [&] { return ba::launch_fwd_ring_bf16(ra, int(p->qtiles.size()), s); });
    } else if (p->dtype == BA_FP8) {
      e = timed("fwd_ring", s, [&] { return ba::launch_fwd_ring_fp8(ra, int(p->qtiles.size()), s); });
    } else {
      const ba::F32Shape sh = f32_shape(*p, scale);
      e = timed("fwd_ring", s, [&] { return ba::launch_fwd_ring_f32(ra, sh, s); });
    }
    if (e != hipSuccess) return hip_fail("fwd_ring launch", e);
    if (has_b) {
      ba::FwdBranchArgs b{};
      b.qb = a->qb;
      b.kb = a->kb;
      b.vb = a->vb;
      b.om = om;
      b.lm = lm;
      b.ob = a->ob;
      b.lseb = a->lseb;
      b.btiles = p->dev.btiles;
      b.branch_off = p->dev.branch_off;
      b.b_anchor = p->dev.b_anchor;
      b.hq = p->hq;
      b.hkv = p->hkv;
      b.G = p->G;
      b.d = p->d;
      b.bidir = p->kind == BA_BRANCH_BLOCK_BIDIR ? 1 : 0;
      b.scale_log2 = scale * ba::kLog2eHost;
      e = timed("fwd_branch_merge", s, [&] {
        return ba::launch_fwd_branch(b, int(p->btiles.size()), p->dtype, p->max_branch_len, s);
      });
      if (e != hipSuccess) return hip_fail("fwd_branch_merge launch", e);
    }
    return BA_OK;
  } catch (...) {
    return fail(BA_E_INVALID, "unexpected error in the forward");
  }
}

}  // namespace

extern "C" ba_status branch_attn_bwd(const ba_plan *p, const ba_bwd_args *a, void *stream) {
  try {
    ba_status st = check_plan(p);
    if (st != BA_OK) return st;
    if (a == nullptr) return fail(BA_E_INVALID, "args is NULL");
    if (!a->q || !a->k || !a->v || !a->o || !a->lse || !a->dout || !a->dq || !a->dk || !a->dv)
      return fail(BA_E_INVALID, "q, k, v, o, lse, dout, dq, dk and dv are required");
    const bool has_b = p->n_branch > 0;
    if (has_b && (!a->qb || !a->kb || !a->vb || !a->ob || !a->lseb || !a->doutb || !a->dqb ||
                  !a->dkb || !a->dvb))
      return fail(BA_E_INVALID, "every branch tensor is required when the plan has branch rows");
    for (const void *ptr :
         {a->q, a->k, a->v, a->qb, a->kb, a->vb, a->o, a->ob, (const void *)a->lse,
          (const void *)a->lseb, a->dout, a->doutb, (const void *)a->dq, (const void *)a->dk,
          (const void *)a->dv, (const void *)a->dqb, (const void *)a->dkb, (const void *)a->dvb,
          (const void *)a->workspace})
      if (!aligned16(ptr)) return fail(BA_E_INVALID, "every pointer must be 16-byte aligned");
    if (a->workspace == nullptr || a->workspace_bytes < p->ws_bwd)
      return fail(BA_E_WORKSPACE, "backward workspace needs " + std::to_string(p->ws_bwd) + " bytes");
    if (!(std::isfinite(a->scale))) return fail(BA_E_INVALID, "scale must be finite");
    const float scale = resolve_scale(a->scale, p->d);
    hipStream_t s = static_cast<hipStream_t>(stream);

    float *ndelta = static_cast<float *>(a->workspace);  // -Delta
    const size_t del_bytes = (size_t(p->n_local + p->n_branch) * p->hq * 4 + 255) & ~size_t(255);
    float *lse2 = reinterpret_cast<float *>(static_cast<char *>(a->workspace) + del_bytes);
    float *dq_local = reinterpret_cast<float *>(static_cast<char *>(a->workspace) + 2 * del_bytes);

    // fp8 plans: the E4M3 q, k, qb, kb are converted to bf16 (exactly) into
    // the workspace, and the bf16 backward runs on those copies, except for
    // the dQ kernel's scores, which take the E4M3 originals
    const void *Q = a->q, *K = a->k, *QB = a->qb, *KB = a->kb;
    const int cdt = p->dtype == BA_FP8 ? int(BA_BF16) : p->dtype;
    if (p->dtype == BA_FP8) {
      auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
      char *c = static_cast<char *>(a->workspace) + 2 * del_bytes +
                al(size_t(p->n_branch) * p->hq * p->d * 4);
      const size_t nq = size_t(p->n_local) * p->hq * p->d, nk = size_t(p->C) * p->n_local * p->hkv * p->d;
      const size_t nqb = size_t(p->n_branch) * p->hq * p->d, nkb = size_t(p->n_branch) * p->hkv * p->d;
      uint16_t *q16 = reinterpret_cast<uint16_t *>(c);
      uint16_t *k16 = reinterpret_cast<uint16_t *>(c + al(nq * 2));
      uint16_t *qb16 = reinterpret_cast<uint16_t *>(c + al(nq * 2) + al(nk * 2));
      uint16_t *kb16 = reinterpret_cast<uint16_t *>(c + al(nq * 2) + al(nk * 2) + al(nqb * 2));
      struct Cv {
        const void *src;
        uint16_t *dst;
        size_t n;
      };
      for (const Cv &cv : {Cv{a->q, q16, nq}, Cv{a->k, k16, nk}, Cv{a->qb, qb16, has_b ? nqb : 0},
                           Cv{a->kb, kb16, has_b ? nkb : 0}}) {
        hipError_t ce = timed("fp8_to_bf16", s, [&] {
          return ba::launch_fp8_to_bf16(static_cast<const uint8_t *>(cv.src), cv.dst, int64_t(cv.n), s);
        });
        if (ce != hipSuccess) return hip_fail("fp8_to_bf16 launch", ce);
      }
      Q = q16;
      K = k16;
      QB = has_b ? qb16 : nullptr;
      KB = has_b ? kb16 : nullptr;
    }

    ba::BwdPreArgs pa{};
    pa.o = a->o;
    pa.ob = a->ob;
    pa.dout = a->dout;
    pa.doutb = a->doutb;
    pa.lse = a->lse;
    pa.lseb = a->lseb;
    pa.bound_main = p->dev.bound_main;
    pa.ndelta = ndelta;
    pa.lse2 = lse2;
    pa.n_local = int32_t(p->n_local);
    pa.n_branch = int32_t(p->n_branch);
    pa.hq = p->hq;
    pa.d = p->d;
    hipError_t e = timed("bwd_pre", s, [&] { return ba::launch_bwd_pre(pa, cdt, s); });
    if (e != hipSuccess) return hip_fail("bwd_pre launch", e);

    if (has_b) {
      ba::BwdBranchArgs b{};
      b.qb = QB;
      b.kb = KB;
      b.vb = a->vb;
      b.doutb = a->doutb;
      b.lseb = a->lseb;
      b.ndelta_b = ndelta + size_t(p->n_local) * p->hq;
      b.dq_local = dq_local;
      b.dkb = a->dkb;
      b.dvb = a->dvb;
      b.btiles = p->dev.btiles;
      b.branch_off = p->dev.branch_off;
      b.b_anchor = p->dev.b_anchor;
      b.hq = p->hq;
      b.hkv = p->hkv;
      b.G = p->G;
      b.d = p->d;
      b.bidir = p->kind == BA_BRANCH_BLOCK_BIDIR ? 1 : 0;
      b.scale = scale;
      b.scale_log2 = scale * ba::kLog2eHost;
      e = timed("bwd_branch", s, [&] {
        return ba::launch_bwd_branch(b, int(p->btiles.size()), cdt, p->max_branch_len, s);
      });
      if (e != hipSuccess) return hip_fail("bwd_branch launch", e);
    }

    ba::BwdDqArgs q{};
    q.q = Q;
    q.qb = QB;
    q.k = K;
    q.v = a->v;
    q.dout = a->dout;
    q.doutb = a->doutb;
    q.lse = a->lse;
    q.lseb = a->lseb;
    q.ndelta = ndelta;
    q.lse2 = lse2;
    q.dq_local = dq_local;
    q.dq = a->dq;
    q.dqb = a->dqb;
    q.qtiles = p->dev.qtiles;
    q.bound_main = p->dev.bound_main;
    q.bound_branch = p->dev.bound_branch;
    q.n_local = int32_t(p->n_local);
    q.n_branch = int32_t(p->n_branch);
    q.hq = p->hq;
    q.hkv = p->hkv;
    q.G = p->G;
    q.log2G = log2i(p->G);
    q.C = p->C;
    q.r = p->r;
    q.d = p->d;
    q.scale = scale;
    q.scale_log2 = scale * ba::kLog2eHost;
    q.runs = ba::uses_run_walk(*p) ? 1 : 0;
    if (p->dtype == BA_FP8) {  // scores on the fp8 matrix cores from the E4M3 originals
      q.q8 = a->q;
      q.qb8 = has_b ? a->qb : nullptr;
      q.k8 = a->k;
    }

    ba::BwdDkdvArgs k{};
    k.q = Q;
    k.qb = QB;
    k.k = K;
    k.v = a->v;
    k.dout = a->dout;
    k.doutb = a->doutb;
    k.lse = a->lse;
    k.lseb = a->lseb;
    k.ndelta = ndelta;
    k.lse2 = lse2;
    k.dk = a->dk;
    k.dv = a->dv;
    k.ktiles = p->dev.ktiles;
    k.bound_main = p->dev.bound_main;
    k.bound_branch = p->dev.bound_branch;
    k.n_local = int32_t(p->n_local);
    k.n_branch = int32_t(p->n_branch);
    k.hq = p->hq;
    k.hkv = p->hkv;
    k.G = p->G;
    k.log2G = log2i(p->G);
    k.d = p->d;
    k.scale = scale;
    k.scale_log2 = scale * ba::kLog2eHost;

    if (cdt == BA_BF16) {
      e = timed("bwd_dq", s, [&] { return ba::launch_bwd_dq_bf16(q, int(p->qtiles.size()), s); });
      if (e != hipSuccess) return hip_fail("bwd_dq launch", e);
      e = timed("bwd_dkdv", s, [&] { return ba::launch_bwd_dkdv_bf16(k, int(p->ktiles.size()), s); });
      if (e != hipSuccess) return hip_fail("bwd_dkdv launch", e);
    } else {
      const ba::F32Shape sh = f32_shape(*p, scale);
      e = timed("bwd_dq", s, [&] { return ba::launch_bwd_dq_f32(q, sh, s); });
      if (e != hipSuccess) return hip_fail("bwd_dq launch", e);
      e = timed("bwd_dkdv", s, [&] { return ba::launch_bwd_dkdv_f32(k, sh, s); });
      if (e != hipSuccess) return hip_fail("bwd_dkdv launch", e);
    }
    return BA_OK;
  } catch (...) {
    return fail(BA_E_INVALID, "unexpected error in branch_attn_bwd");
  }
}

extern "C" ba_status ba_qkv_project(const ba_plan *p, const ba_proj_args *a, void *stream) {
  try {
    ba_status st = check_plan(p);
    if (st != BA_OK) return st;
    if (a == nullptr) return fail(BA_E_INVALID, "args is NULL");
    if (p->dtype != BA_BF16 || p->d != 128)
      return fail(BA_E_UNSUPPORTED, "the projection supports bf16 plans with d == 128");
    if (a->target != 0 && a->target != 1) return fail(BA_E_INVALID, "target must be 0 or 1");
    if (a->hidden < 64 || a->hidden % 64 != 0)
      return fail(BA_E_INVALID, "hidden must be a positive multiple of 64");
    // a 256-row tile of x (2 bytes per element) must stay below 4 GiB: the
    // tile loads address it with 32-bit offsets
    if (int64_t(a->hidden) * 2 * 256 >= (int64_t(1) << 32))
      return fail(BA_E_UNSUPPORTED, "hidden too large for 32-bit tile offsets");
    if (!std::isfinite(a->rope_theta) || !std::isfinite(a->norm_eps) || a->norm_eps < 0.f)
      return fail(BA_E_INVALID, "rope_theta must be finite and norm_eps finite and >= 0");
    if ((a->q_norm == nullptr) != (a->k_norm == nullptr))
      return fail(BA_E_INVALID, "give both q_norm and k_norm or neither");
    int64_t rows = 0;
    if (a->target == 0) {
      if (a->step != -1) return fail(BA_E_INVALID, "step applies to branch rows only");
      rows = p->n_local;
    } else if (a->step == -1) {
      rows = p->n_branch;
    } else {
      if (p->kind != BA_BRANCH_TTT)
        return fail(BA_E_INVALID, "a step pass needs a TTT plan (every anchor has every step)");
      if (a->step < 0 || a->step >= p->depth_or_block)
        return fail(BA_E_INVALID, "step must be -1 or in 0 .. depth - 1");
      rows = int64_t(p->anchor_row.size());
    }
    if (rows == 0) return BA_OK;
    if (!a->x || !a->w || !a->q || !a->k || !a->v)
      return fail(BA_E_INVALID, "x, w, q, k and v are required");
    for (const void *ptr : {a->x, a->w, (const void *)a->q, (const void *)a->k, (const void *)a->v,
                            a->q_norm, a->k_norm})
      if (!aligned16(ptr)) return fail(BA_E_INVALID, "every pointer must be 16-byte aligned");
    if (rows * int64_t(a->hidden) * 2 > (int64_t(1) << 40))
      return fail(BA_E_UNSUPPORTED, "x too large");
    ba::ProjArgs k{};
    k.x = a->x;
    k.w = a->w;
    k.q_norm = a->q_norm;
    k.k_norm = a->k_norm;
    k.q = a->q;
    k.k = a->k;
    k.v = a->v;
    k.bound_main = p->dev.bound_main;
    k.branch_off = p->dev.branch_off;
    k.b_anchor = p->dev.b_anchor;
    k.anchor_pos = p->dev.anchor_pos;
    k.nrows = int32_t(rows);
    k.hidden = a->hidden;
    k.hq = p->hq;
    k.hkv = p->hkv;
    k.target = a->target;
    k.step = a->step;
    k.rope = a->rope_theta > 0.f ? 1 : 0;
    k.eps = a->norm_eps;
    for (int j = 0; j < 64; ++j)
      k.inv_freq[j] = k.rope ? std::pow(double(a->rope_theta), -2.0 * j / 128.0) : 0.0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("qkv_project", s, [&] { return ba::launch_qkv_project(k, s); });
    if (e != hipSuccess) return hip_fail("qkv_project launch", e);
    return BA_OK;
  } catch (...) {
    return fail(BA_E_INVALID, "unexpected error in ba_qkv_project");
  }
}

extern "C" ba_status ba_profile_enable(int32_t on, int32_t max_launches) {
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (!on) {
    P.on = false;
    return BA_OK;
  }
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(BA_E_INVALID, "max_launches must be in 1..2^20");
  while (P.ev0.size() < size_t(max_launches)) {
    hipEvent_t e0, e1;
    hipError_t e = hipEventCreate(&e0);
    if (e != hipSuccess) return hip_fail("hipEventCreate", e);
    e = hipEventCreate(&e1);
    if (e != hipSuccess) {
      (void)hipEventDestroy(e0);
      return hip_fail("hipEventCreate", e);
    }
    P.ev0.push_back(e0);
    P.ev1.push_back(e1);
    P.names.emplace_back();
  }
  P.used = 0;
  P.on = true;
  return BA_OK;
}

extern "C" ba_status ba_profile_read(ba_kernel_time *out, int32_t max_entries, int32_t *n_entries) {
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (n_entries == nullptr) return fail(BA_E_INVALID, "n_entries is NULL");
  std::vector<ba_kernel_time> agg;
  for (size_t i = 0; i < P.used; ++i) {
    hipError_t e = hipEventSynchronize(P.ev1[i]);
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, P.ev0[i], P.ev1[i]);
    if (e != hipSuccess) return hip_fail("hipEventElapsedTime", e);
    size_t k = 0;
    while (k < agg.size() && std::strncmp(agg[k].name, P.names[i].c_str(), 31) != 0) ++k;
    if (k == agg.size()) {
      ba_kernel_time t{};
      std::strncpy(t.name, P.names[i].c_str(), 31);
      agg.push_back(t);
    }
    agg[k].launches += 1;
    agg[k].total_ms += ms;
  }
  P.used = 0;
  *n_entries = int32_t(agg.size());
  if (out != nullptr)
    for (size_t k = 0; k < agg.size() && int32_t(k) < max_entries; ++k) out[k] = agg[k];
  return BA_OK;
}
