// C-ABI entry points of the attention library: validation, stride set-up
// and kernel dispatch.  No allocation, no global state, no printing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "attn_kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Strides {
  int64_t sb, sh, sn;
};

Strides strides_for(attn_layout layout, int64_t H, int64_t N, int64_t d) {
  if (layout == ATTN_BHND) return {H * N * d, N * d, d};
  return {N * H * d, d, H * d};
}

float resolve_scale(const attn_params* p) {
  const float s = p->scale;
  if (!(s > 0.0f)) return 1.0f / sqrtf((float)p->d);
  return s;
}

constexpr float kLog2eF = 1.4426950408889634f;
constexpr int64_t kLocalMaxPositions = int64_t(1) << 29;   // Nq + Nk bound of local calls

bool has_window(const attn_params* p) {
  return p->window != 0 && (p->window_left >= 0 || p->window_right >= 0);
}
// window or grid: the local kernels
bool is_local(const attn_params* p) { return has_window(p) || p->grid_cols > 0; }

// Checks of the local fields shared by every entry point.
attn_status validate_local(const attn_params* p) {
  if (p->grid_cols < 0) return ATTN_EINVAL;
  if (p->grid_cols > 0 && (p->nbr_rows < 1 || p->nbr_cols < 1)) return ATTN_EINVAL;
  if (!(p->softcap >= 0.0f) || !isfinite(p->softcap)) return ATTN_EINVAL;
  if (p->softcap > 0.0f && !isfinite(2.0f * resolve_scale(p) * kLog2eF / p->softcap))
    return ATTN_EINVAL;
  if ((has_window(p) || p->grid_cols > 0) && (int64_t)p->Nq + p->Nk >= kLocalMaxPositions)
    return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

// Window and grid in kernel form: an open side becomes Nq + Nk (beyond every
// position), causal caps the right side at 0, and the grid's column count
// and row radius are clamped to values that leave the relation unchanged
// but keep the kernels' index arithmetic inside int32.
attn::LocalVis local_vis(const attn_params* p) {
  const int32_t open = p->Nq + p->Nk;
  attn::LocalVis L = {};
  L.win_l = open;
  L.win_r = open;
  if (p->window) {
    if (p->window_left >= 0) L.win_l = p->window_left < open ? p->window_left : open;
    if (p->window_right >= 0) L.win_r = p->window_right < open ? p->window_right : open;
  }
  if (p->causal && L.win_r > 0) L.win_r = 0;
  if (p->grid_cols > 0) {
    // positions are < open, so with cols >= open every position is in row 0
    // and its column is the position itself, as with the caller's value
    L.cols = p->grid_cols < open ? p->grid_cols : open;
    const int32_t rows = open / L.cols + 2;   // exceeds any row difference
    L.nbr_r = p->nbr_rows < rows ? p->nbr_rows : rows;
    L.nbr_c = p->nbr_cols < L.cols ? p->nbr_cols : L.cols;
  }
  return L;
}

void softcap_consts(const attn_params* p, float* a, float* c2) {
  *a = *c2 = 0.0f;
  if (p->softcap > 0.0f) {
    *a = p->softcap * kLog2eF;
    *c2 = 2.0f * resolve_scale(p) * kLog2eF / p->softcap;
  }
}

}  // namespace

extern "C" {

attn_status attn_validate(const attn_params* p, int for_backward) {
  if (!p) return ATTN_EINVAL;
  if (p->B < 0 || p->Nq < 0 || p->Nk < 0 || p->Hq < 1 || p->Hkv < 1) return ATTN_EINVAL;
  if (p->Hq % p->Hkv != 0) return ATTN_EINVAL;
  if (p->d < 1) return ATTN_EINVAL;
  if (p->dtype != ATTN_FP32 && p->dtype != ATTN_FP16 && p->dtype != ATTN_BF16) return ATTN_EINVAL;
  if (p->layout != ATTN_BHND && p->layout != ATTN_BNHD) return ATTN_EINVAL;
  if (p->causal && p->Nq != p->Nk) return ATTN_EINVAL;
  if (is_local(p) && p->Nq != p->Nk) return ATTN_EINVAL;
  if (p->mask && (p->mask_sb < 0 || p->mask_sh < 0 || p->mask_sq < 0)) return ATTN_EINVAL;
  const attn_status sl = validate_local(p);
  if (sl != ATTN_OK) return sl;
  if (p->d < 8 || p->d > 128 || p->d % 8 != 0) return ATTN_EUNSUPPORTED;
  (void)for_backward;   // the backward takes everything the forward takes
  return ATTN_OK;
}

attn_status attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, void* o,
                     float* lse, void* stream) {
  const attn_status st = attn_validate(p, 0);
  if (st != ATTN_OK) return st;
  if (p->B == 0 || p->Nq == 0) return ATTN_OK;  // nothing to compute
  // k and v may be null when there are no keys (every row is then fully masked)
  if (!q || !o || !lse || (p->Nk > 0 && (!k || !v))) return ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_EALIGN;
  if (p->mask && (reinterpret_cast<uintptr_t>(p->mask) & 3u)) return ATTN_EALIGN;
  if (p->kv_lens && (reinterpret_cast<uintptr_t>(p->kv_lens) & 3u)) return ATTN_EALIGN;

  attn::FwdArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.mask = p->mask;
  a.kv_lens = p->kv_lens;
  const Strides sq = strides_for(p->layout, p->Hq, p->Nq, p->d);
  const Strides sk = strides_for(p->layout, p->Hkv, p->Nk, p->d);
  a.q_sb = sq.sb; a.q_sh = sq.sh; a.q_sn = sq.sn;
  a.o_sb = sq.sb; a.o_sh = sq.sh; a.o_sn = sq.sn;
  a.k_sb = sk.sb; a.k_sh = sk.sh; a.k_sn = sk.sn;
  a.v_sb = sk.sb; a.v_sh = sk.sh; a.v_sn = sk.sn;
  a.m_sb = p->mask_sb; a.m_sh = p->mask_sh; a.m_sq = p->mask_sq;
  a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.d = p->d;
  a.group = p->Hq / p->Hkv;
  a.c = resolve_scale(p) * kLog2eF;
  a.loc = local_vis(p);
  softcap_consts(p, &a.cap_a, &a.cap_c2);
  attn::FwdMode m;
  m.local = is_local(p);
  m.causal = p->causal != 0 && !m.local;   // folded into the window when local
  m.mask = p->mask != nullptr;
  m.softcap = p->softcap > 0.0f;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->dtype == ATTN_FP32)
    e = attn::launch_fwd32(a, m, s);
  else
    e = attn::launch_fwd16(a, p->dtype == ATTN_BF16, m, s);
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: D [B,Hq,ld] | nl2 [B,Hq,ld] | (kv_chunks > 1) partial
// dK and dV, [kv_chunks, B, Hkv, Nk, d] fp32 each | (bf16 inputs) fp16
// copies of q, dout and k in their own layout, then the pre-pass maxima
// [kBwdAmaxBlocks][4] and the 4 operand scales; ld = Nq rounded up to 128.
struct BwdWorkspace {
  size_t rows, part, cq, ck, amax, total;
  int chunks, ld;
};

BwdWorkspace bwd_workspace(const attn_params* p) {
  BwdWorkspace w;
  // the fp32 dK/dV kernel sums all q-heads of a kv-head itself (no partials)
  w.chunks = p->dtype == ATTN_FP32 ? 1 : attn::bwd_kv_chunks(p->B, p->Hkv, p->Nk, p->Hq / p->Hkv);
  w.ld = (p->Nq + 127) / 128 * 128;
  w.rows = align256((size_t)p->B * p->Hq * w.ld * sizeof(float));
  w.part = w.chunks > 1 ? align256((size_t)w.chunks * p->B * p->Hkv * p->Nk * p->d * sizeof(float)) : 0;
  // bf16 inputs: fp16 copies of q and dout (cq bytes each) and of k (ck)
  const bool cvt = p->dtype == ATTN_BF16;
  w.cq = cvt ? align256((size_t)p->B * p->Hq * p->Nq * p->d * 2) : 0;
  w.ck = cvt ? align256((size_t)p->B * p->Hkv * p->Nk * p->d * 2) : 0;
  w.amax = cvt ? align256((size_t)attn::kBwdAmaxBlocks * 4 * sizeof(float)) + 256 : 0;
  w.total = 2 * w.rows + 2 * w.part + 2 * w.cq + w.ck + w.amax;
  return w;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(const attn_params* p) {
  if (attn_validate(p, 1) != ATTN_OK) return 0;
  const size_t t = bwd_workspace(p).total;
  return t > 0 ? t : 256;
}

attn_status attn_bwd(const attn_params* p, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout, void* dq, void* dk,
                     void* dv, attn_dtype grad_dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const attn_status st = attn_validate(p, 1);
  if (st != ATTN_OK) return st;
  if (grad_dtype != ATTN_FP32 && grad_dtype != p->dtype) return ATTN_EINVAL;
  if (p->B == 0 || (p->Nq == 0 && p->Nk == 0)) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_EINVAL;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, workspace};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return ATTN_EALIGN;
  if (p->kv_lens && (reinterpret_cast<uintptr_t>(p->kv_lens) & 3u)) return ATTN_EALIGN;
  if (p->mask && (reinterpret_cast<uintptr_t>(p->mask) & 3u)) return ATTN_EALIGN;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(p)) return ATTN_EWORKSPACE;

  attn::BwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  const BwdWorkspace ws = bwd_workspace(p);
  char* wsp = static_cast<char*>(workspace);
  a.delta = reinterpret_cast<float*>(wsp);
  a.nl2 = reinterpret_cast<float*>(wsp + ws.rows);
  a.part_dk = ws.part ? reinterpret_cast<float*>(wsp + 2 * ws.rows) : nullptr;
  a.part_dv = ws.part ? reinterpret_cast<float*>(wsp + 2 * ws.rows + ws.part) : nullptr;
  if (ws.cq) {
    char* c = wsp + 2 * ws.rows + 2 * ws.part;
    a.q16 = c;
    a.do16 = c + ws.cq;
    a.k16 = c + 2 * ws.cq;
    a.amax_part = reinterpret_cast<float*>(c + 2 * ws.cq + ws.ck);
    a.escale = reinterpret_cast<float*>(c + 2 * ws.cq + ws.ck + ws.amax - 256);
  } else {
    a.q16 = q;
    a.do16 = dout;
    a.k16 = k;
  }
  a.kv_chunks = ws.chunks;
  a.ld_rows = ws.ld;
  a.kv_lens = p->kv_lens;
  a.mask = p->mask;
  a.m_sb = p->mask_sb; a.m_sh = p->mask_sh; a.m_sq = p->mask_sq;
  const Strides sq = strides_for(p->layout, p->Hq, p->Nq, p->d);
  const Strides sk = strides_for(p->layout, p->Hkv, p->Nk, p->d);
  a.q_sb = sq.sb; a.q_sh = sq.sh; a.q_sn = sq.sn;
  a.k_sb = sk.sb; a.k_sh = sk.sh; a.k_sn = sk.sn;
  a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.d = p->d;
  a.group = p->Hq / p->Hkv;
  a.scale = resolve_scale(p);
  a.c = a.scale * kLog2eF;
  a.grad_f32 = grad_dtype == ATTN_FP32 ? 1 : 0;
  a.loc = local_vis(p);
  softcap_consts(p, &a.cap_a, &a.cap_c2);
  attn::FwdMode m;
  m.local = is_local(p);
  m.causal = p->causal != 0 && !m.local;   // folded into the window when local
  m.mask = p->mask != nullptr;
  m.softcap = p->softcap > 0.0f;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = p->dtype == ATTN_FP32 ? attn::launch_bwd32(a, m, s)
                                             : attn::launch_bwd16(a, p->dtype == ATTN_BF16, m, s);
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // extern "C"

namespace {

// Validation of a decode call: attn_validate's rules, except that causal and
// the window (bottom-right aligned) do not need Nq == Nk; 16-bit dtypes, no
// mask, no grid.
attn_status validate_decode(const attn_params* p) {
  if (!p) return ATTN_EINVAL;
  attn_params c = *p;
  c.causal = 0;
  c.window = 0;
  const int grid = c.grid_cols;
  c.grid_cols = 0;
  attn_status st = attn_validate(&c, 0);
  if (st != ATTN_OK) return st;
  if (grid < 0) return ATTN_EINVAL;
  // positions and window bounds stay far inside int32 (see local_vis)
  if ((int64_t)p->Nq + p->Nk >= kLocalMaxPositions) return ATTN_EUNSUPPORTED;
  if (p->dtype == ATTN_FP32 || p->mask || grid > 0) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

// Keys a decode call may read per batch: with a bounded left window only the
// last Nq + window_left keys of each batch's L are visible to any query.
int decode_span(const attn_params* p) {
  if (has_window(p) && p->window_left >= 0 && (int64_t)p->Nq + p->window_left < p->Nk)
    return p->Nq + p->window_left;
  return p->Nk;
}

struct DecodeWorkspace {
  int split_keys, n_splits;
  size_t part_o, total;
};

DecodeWorkspace decode_workspace(const attn_params* p) {
  DecodeWorkspace w;
  const int rows = (p->Hq / p->Hkv) * p->Nq;
  attn::decode_split(p->B, p->Hkv, rows, decode_span(p), &w.split_keys, &w.n_splits);
  const size_t nrow = (size_t)p->B * p->Hq * p->Nq;
  w.part_o = align256((size_t)w.n_splits * nrow * p->d * sizeof(float));
  w.total = w.part_o + align256((size_t)w.n_splits * nrow * sizeof(float));
  return w;
}

}  // namespace

extern "C" {

size_t attn_decode_workspace_bytes(const attn_params* p) {
  if (validate_decode(p) != ATTN_OK) return 0;
  const size_t t = decode_workspace(p).total;
  return t > 0 ? t : 256;
}

}  // extern "C"

namespace {

// Argument checks of a decode call that need no workspace.
attn_status check_decode_args(const attn_params* p, const void* q, const void* k, const void* v,
                              const void* o, const float* lse) {
  if (!q || !o || !lse) return ATTN_EINVAL;
  if (p->Nk > 0 && (!k || !v)) return ATTN_EINVAL;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return ATTN_EALIGN;
  if (p->kv_lens && (reinterpret_cast<uintptr_t>(p->kv_lens) & 3u)) return ATTN_EALIGN;
  return ATTN_OK;
}

// The decode launch on a checked call with a workspace of at least
// decode_workspace(p).total bytes.
attn_status run_decode(const attn_params* p, const void* q, const void* k, const void* v,
                       void* o, float* lse, void* workspace, void* stream) {
  const DecodeWorkspace ws = decode_workspace(p);
  attn::DecodeArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.kv_lens = p->kv_lens;
  char* wsp = static_cast<char*>(workspace);
  a.part_o = reinterpret_cast<float*>(wsp);
  a.part_lse = reinterpret_cast<float*>(wsp + ws.part_o);
  const Strides sq = strides_for(p->layout, p->Hq, p->Nq, p->d);
  const Strides sk = strides_for(p->layout, p->Hkv, p->Nk, p->d);
  a.q_sb = sq.sb; a.q_sh = sq.sh; a.q_sn = sq.sn;
  a.k_sb = sk.sb; a.k_sh = sk.sh; a.k_sn = sk.sn;
  a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.d = p->d;
  a.group = p->Hq / p->Hkv;
  a.rows = a.group * p->Nq;
  a.n_rb = (a.rows + 31) / 32;
  a.split_keys = ws.split_keys;
  a.n_splits = ws.n_splits;
  a.causal = p->causal ? 1 : 0;
  a.c = resolve_scale(p) * kLog2eF;
  {
    attn_params c = *p;
    c.grid_cols = 0;
    const attn::LocalVis L = local_vis(&c);   // open sides Nq + Nk, causal folded in
    a.win_l = L.win_l;
    a.win_r = L.win_r;
  }
  softcap_consts(p, &a.cap_a, &a.cap_c2);
  const hipError_t e = attn::launch_decode(a, p->dtype == ATTN_BF16, p->softcap > 0.0f,
                                           reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // namespace

// Scratch of attn_decode_static: one copy per GPU, for callers that cannot
// allocate.  Host code never uses this name as an address: it takes the
// device address of the current GPU's copy from hipGetSymbolAddress, once
// per device (scratch_ptr below).
static __device__ __align__(256) char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current GPU's scratch (nullptr on failure).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

attn_status attn_decode(const attn_params* p, const void* q, const void* k, const void* v,
                        void* o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const attn_status st = validate_decode(p);
  if (st != ATTN_OK) return st;
  if (p->B == 0 || p->Nq == 0) return ATTN_OK;
  const attn_status ca = check_decode_args(p, q, k, v, o, lse);
  if (ca != ATTN_OK) return ca;
  if (workspace && !aligned16(workspace)) return ATTN_EALIGN;
  if (!workspace || workspace_bytes < attn_decode_workspace_bytes(p)) return ATTN_EWORKSPACE;
  return run_decode(p, q, k, v, o, lse, workspace, stream);
}

attn_status attn_decode_static(const attn_params* p, const void* q, const void* k,
                               const void* v, void* o, float* lse, void* stream) {
  const attn_status st = validate_decode(p);
  if (st != ATTN_OK) return st;
  if (p->B == 0 || p->Nq == 0) return ATTN_OK;
  const attn_status ca = check_decode_args(p, q, k, v, o, lse);
  if (ca != ATTN_OK) return ca;
  if (decode_workspace(p).total > (size_t)ATTN_DECODE_SCRATCH_BYTES) return ATTN_ESCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return ATTN_EHIP;
  return run_decode(p, q, k, v, o, lse, ws, stream);
}

}  // extern "C"

namespace {

attn_status validate_fp8(const attn_params* p) {
  if (!p) return ATTN_EINVAL;
  const attn_status st = attn_validate(p, 0);
  if (st != ATTN_OK) return st;
  if (p->d % 16 != 0) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

int64_t round64(int64_t n) { return (n + 63) / 64 * 64; }

}  // namespace

extern "C" {

attn_status attn_quantize_fp8(const attn_params* p, const void* q, const void* k, const void* v,
                              void* q8, void* k8, void* vt8, float* q_scale, float* k_scale,
                              float* v_scale, void* stream) {
  const attn_status st = validate_fp8(p);
  if (st != ATTN_OK) return st;
  if (p->B == 0) return ATTN_OK;
  const bool has_q = p->Nq > 0, has_k = p->Nk > 0;
  if ((has_q && (!q || !q8 || !q_scale)) || (has_k && (!k || !v || !k8 || !vt8 || !k_scale || !v_scale)))
    return ATTN_EINVAL;
  const void* ptrs[] = {q, k, v, q8, k8, vt8, q_scale, k_scale, v_scale};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return ATTN_EALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int in_dtype = p->dtype == ATTN_BF16 ? 2 : (p->dtype == ATTN_FP16 ? 1 : 0);
  auto one = [&](const void* x, void* out, float* scale, int H, int N, bool transpose) {
    attn::QuantArgs a = {};
    const Strides sx = strides_for(p->layout, H, N, p->d);
    a.x = x;
    a.out = out;
    a.scale = scale;
    a.x_sb = sx.sb; a.x_sh = sx.sh; a.x_sn = sx.sn;
    a.o_sb = sx.sb; a.o_sh = sx.sh; a.o_sn = sx.sn;   // 1-byte codes: same numbers
    a.o_ld = round64(N);
    a.B = p->B; a.H = H; a.N = N; a.d = p->d;
    a.nblk = (N + 63) / 64;
    a.transpose = transpose ? 1 : 0;
    return attn::launch_fp8_quant(a, in_dtype, s);
  };
  hipError_t e = hipSuccess;
  if (has_q) e = one(q, q8, q_scale, p->Hq, p->Nq, false);
  if (e == hipSuccess && has_k) e = one(k, k8, k_scale, p->Hkv, p->Nk, false);
  if (e == hipSuccess && has_k) e = one(v, vt8, v_scale, p->Hkv, p->Nk, true);
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

attn_status attn_fwd_fp8(const attn_params* p, const void* q8, const void* k8, const void* vt8,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         void* o, float* lse, void* stream) {
  const attn_status st = validate_fp8(p);
  if (st != ATTN_OK) return st;
  if (p->dtype == ATTN_FP32 || p->mask || is_local(p) || p->softcap > 0.0f)
    return ATTN_EUNSUPPORTED;
  if (p->B == 0 || p->Nq == 0) return ATTN_OK;
  if (!q8 || !q_scale || !o || !lse) return ATTN_EINVAL;
  if (p->Nk > 0 && (!k8 || !vt8 || !k_scale || !v_scale)) return ATTN_EINVAL;
  const void* ptrs[] = {q8, k8, vt8, q_scale, k_scale, v_scale, o, lse};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return ATTN_EALIGN;
  if (p->kv_lens && (reinterpret_cast<uintptr_t>(p->kv_lens) & 3u)) return ATTN_EALIGN;
  attn::Fp8Args a = {};
  a.q = static_cast<const uint8_t*>(q8);
  a.k = static_cast<const uint8_t*>(k8);
  a.vt = static_cast<const uint8_t*>(vt8);
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.o = o;
  a.lse = lse;
  a.kv_lens = p->kv_lens;
  const Strides sq = strides_for(p->layout, p->Hq, p->Nq, p->d);
  const Strides sk = strides_for(p->layout, p->Hkv, p->Nk, p->d);
  a.q_sb = sq.sb; a.q_sh = sq.sh; a.q_sn = sq.sn;
  a.o_sb = sq.sb; a.o_sh = sq.sh; a.o_sn = sq.sn;
  a.k_sb = sk.sb; a.k_sh = sk.sh; a.k_sn = sk.sn;
  a.vt_ld = round64(p->Nk);
  a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.Nq = p->Nq; a.Nk = p->Nk; a.d = p->d;
  a.group = p->Hq / p->Hkv;
  a.nqs = (p->Nq + 63) / 64;
  a.nks = (p->Nk + 63) / 64;
  a.c = resolve_scale(p) * kLog2eF;
  const hipError_t e = attn::launch_fwd_fp8(a, p->dtype == ATTN_BF16, p->causal != 0,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid shape or parameter";
    case ATTN_EUNSUPPORTED: return "unsupported configuration";
    case ATTN_EALIGN: return "pointer not 16-byte aligned";
    case ATTN_EWORKSPACE: return "workspace missing or too small";
    case ATTN_ESCRATCH: return "call needs more scratch than attn_decode_static's fixed buffer holds";
    case ATTN_EHIP: return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
