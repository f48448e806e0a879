// C-ABI entry points of the attention library: validation, stride set-up
// and kernel dispatch.  No allocation, no global state, no printing.
#include <math.h>
#include <stdint.h>

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
  if (p->mask && (p->mask_sb < 0 || p->mask_sh < 0 || p->mask_sq < 0)) return ATTN_EINVAL;
  if (p->d < 8 || p->d > 128 || p->d % 8 != 0) return ATTN_EUNSUPPORTED;
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
  a.c = resolve_scale(p) * 1.4426950408889634f;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->dtype == ATTN_FP32)
    e = attn::launch_fwd32(a, p->causal != 0, p->mask != nullptr, s);
  else
    e = attn::launch_fwd16(a, p->dtype == ATTN_BF16, p->causal != 0, p->mask != nullptr, s);
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout: D [B,Hq,ld] | nl2 [B,Hq,ld] | (kv_chunks > 1) partial
// dK and dV, [kv_chunks, B, Hkv, Nk, d] fp32 each | (bf16 inputs) fp16
// copies of q, dout and k in their own layout; ld = Nq rounded up to 128.
struct BwdWorkspace {
  size_t rows, part, cq, ck, total;
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
  w.total = 2 * w.rows + 2 * w.part + 2 * w.cq + w.ck;
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
  a.c = a.scale * 1.4426950408889634f;
  a.grad_f32 = grad_dtype == ATTN_FP32 ? 1 : 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = p->dtype == ATTN_FP32
                           ? attn::launch_bwd32(a, p->causal != 0, s)
                           : attn::launch_bwd16(a, p->dtype == ATTN_BF16, p->causal != 0, s);
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // extern "C"

namespace {

// Validation of a decode call: attn_validate's rules, except that causal
// (bottom-right aligned) does not need Nq == Nk; 16-bit dtypes, no mask.
attn_status validate_decode(const attn_params* p) {
  if (!p) return ATTN_EINVAL;
  attn_params c = *p;
  c.causal = 0;
  const attn_status st = attn_validate(&c, 0);
  if (st != ATTN_OK) return st;
  if (p->dtype == ATTN_FP32 || p->mask) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

struct DecodeWorkspace {
  int split_keys, n_splits;
  size_t part_o, total;
};

DecodeWorkspace decode_workspace(const attn_params* p) {
  DecodeWorkspace w;
  const int rows = (p->Hq / p->Hkv) * p->Nq;
  attn::decode_split(p->B, p->Hkv, rows, p->Nk, &w.split_keys, &w.n_splits);
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

attn_status attn_decode(const attn_params* p, const void* q, const void* k, const void* v,
                        void* o, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  const attn_status st = validate_decode(p);
  if (st != ATTN_OK) return st;
  if (p->B == 0 || p->Nq == 0) return ATTN_OK;
  if (!q || !o || !lse) return ATTN_EINVAL;
  if (p->Nk > 0 && (!k || !v)) return ATTN_EINVAL;
  const void* ptrs[] = {q, k, v, o, lse, workspace};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return ATTN_EALIGN;
  if (p->kv_lens && (reinterpret_cast<uintptr_t>(p->kv_lens) & 3u)) return ATTN_EALIGN;
  if (!workspace || workspace_bytes < attn_decode_workspace_bytes(p)) return ATTN_EWORKSPACE;

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
  a.c = resolve_scale(p) * 1.4426950408889634f;
  const hipError_t e = attn::launch_decode(a, p->dtype == ATTN_BF16,
                                           reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid shape or parameter";
    case ATTN_EUNSUPPORTED: return "unsupported configuration";
    case ATTN_EALIGN: return "pointer not 16-byte aligned";
    case ATTN_EWORKSPACE: return "backward workspace missing or too small";
    case ATTN_EHIP: return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
