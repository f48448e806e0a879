// Internal interface between the C-ABI host code and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "local_mask.h"

namespace attn {

// Kernel arguments of the forward pass.  Strides are in elements; d is the
// contiguous dimension of every tensor.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* mask;
  const int32_t* kv_lens;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t m_sb, m_sh, m_sq;
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int32_t group;         // Hq / Hkv
  int32_t nqb;           // query blocks per head (set by the launcher)
  int32_t total_blocks;  // B * Hq * nqb (set by the launcher)
  float c;               // scale * log2(e)
  LocalVis loc;          // window / grid (local launches only)
  float cap_a, cap_c2;   // soft cap: cap * log2(e), 2 * scale * log2(e) / cap
};

// Kernel arguments of the backward pass (16-bit inputs).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  // fp16 copies of q, dout and k (same strides) for the products that take
  // P or dS; for fp16 inputs they are q, dout and k themselves
  const void* q16;
  const void* do16;
  const void* k16;
  // bf16 inputs: per-block largest magnitudes of q, k, v, dout
  // ([amax_blocks][4]) and the power-of-two operand scales derived from them
  // (sq, sk, sv, sdo; see BwdScales); null for fp16 inputs (all scales 1)
  float* amax_part;
  float* escale;
  int32_t amax_blocks;
  void* dq;
  void* dk;
  void* dv;
  float* delta;          // [B, Hq, ld_rows] workspace: D = rowsum(P * dP)
  float* nl2;            // [B, Hq, ld_rows] workspace: -lse * log2(e)
  float* part_dk;        // [kv_chunks, B, Hkv, Nk, d] workspace (kv_chunks > 1)
  float* part_dv;
  const int32_t* kv_lens;
  const float* mask;     // optional additive mask, element (b,h,i,j) at
  int64_t m_sb, m_sh, m_sq;   // mask[b*m_sb + h*m_sh + i*m_sq + j]
  int64_t q_sb, q_sh, q_sn;   // q, o, dout, dq share these
  int64_t k_sb, k_sh, k_sn;   // k, v, dk, dv share these
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int32_t group;
  float scale;           // softmax scale
  float c;               // scale * log2(e)
  int32_t grad_f32;      // 1: dq/dk/dv are fp32, 0: input dtype
  int32_t kv_chunks;     // q-head chunks per kv-head in the dK/dV pass
  int32_t ld_rows;       // row stride of delta / nl2 per (b, h): Nq rounded up to 128
  LocalVis loc;          // window / grid (local launches only)
  float cap_a, cap_c2;   // soft cap (see FwdArgs)
};

// Kernel arguments of the split-KV decode (attn_decode.hip).  The Nq new
// queries of the `group` q-heads that share a kv-head are stacked into
// rows = group * Nq rows (row r: q-head g*group + r / Nq, query r % Nq), and
// the keys are cut into n_splits ranges of split_keys keys; each (batch,
// kv-head, 32-row block, key range) yields a partial O and LSE, which the
// merge kernel combines.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* kv_lens;
  float* part_o;         // [n_splits, B, Hq, Nq, d] fp32 (workspace)
  float* part_lse;       // [n_splits, B, Hq, Nq] fp32 (workspace)
  int64_t q_sb, q_sh, q_sn;   // q and o share these
  int64_t k_sb, k_sh, k_sn;   // k and v share these
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int32_t group;         // Hq / Hkv
  int32_t rows;          // group * Nq
  int32_t n_rb;          // 32-row blocks: ceil(rows / 32)
  int32_t split_keys;    // keys per split (a multiple of 32)
  int32_t n_splits;      // ceil(Nk / split_keys)
  int32_t causal;        // 1: query i sees keys j <= L - Nq + i (L = the batch's key count)
  float c;               // scale * log2(e)
  // query i (position p = L - Nq + i) sees keys p - win_l .. p + win_r; an
  // open side is Nq + Nk, and causal is folded in as win_r <= 0
  int32_t win_l, win_r;
  float cap_a, cap_c2;   // soft cap (see FwdArgs), used when soft-capped
};

// Kernel arguments of the FP8 forward (attn_fp8.hip).  q, k hold E4M3 codes
// in the layout of the call (strides in elements = bytes); vt holds V
// transposed, [B, Hkv, d, vt_ld] with keys contiguous; every scale array
// has one fp32 value per 64 rows of a (batch, head).
struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* vt;
  const float* q_scale;  // [B, Hq, nqs]
  const float* k_scale;  // [B, Hkv, nks]
  const float* v_scale;  // [B, Hkv, nks]
  void* o;
  float* lse;
  const int32_t* kv_lens;
  int64_t q_sb, q_sh, q_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t vt_ld;         // Nk rounded up to 64
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int32_t group;
  int32_t nqs, nks;      // 64-row blocks per head of q and of k / v
  int32_t nqb, total_blocks;  // set by the launcher
  float c;               // scale * log2(e)
};

// Kernel arguments of the FP8 block quantiser: x [B, H, N, d] in a layout
// (element strides) -> codes (natural: byte strides o_*; transposed:
// [B, H, d, o_ld]) and one scale per 64 rows.
struct QuantArgs {
  const void* x;
  void* out;
  float* scale;          // [B, H, nblk]
  int64_t x_sb, x_sh, x_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t o_ld;
  int32_t B, H, N, d, nblk;
  int32_t transpose;
};

hipError_t launch_fp8_quant(const QuantArgs& a, int in_dtype, hipStream_t st);
hipError_t launch_fwd_fp8(const Fp8Args& a, bool out_bf16, bool causal, hipStream_t st);

// Split of the decode's keys, shared by the workspace sizing and the launch.
void decode_split(int B, int Hkv, int rows, int Nk, int* split_keys, int* n_splits);
hipError_t launch_decode(const DecodeArgs& a, bool is_bf16, bool softcap, hipStream_t st);

// Work split of the backward, shared by the workspace sizing and the launch.
constexpr int kBwdKeysPerBlock = 128;   // keys per dK/dV work-group
constexpr int kBwdAmaxBlocks = 2048;    // work-groups of the bf16 -> fp16 pre-pass
int bwd_kv_chunks(int B, int Hkv, int Nk, int group);

// Variant switches of a forward launch.
struct FwdMode {
  bool causal;    // causal, outside local launches
  bool mask;      // additive mask
  bool local;     // window and/or grid in a.loc (causal folded into it)
  bool softcap;   // soft cap (a.cap_a, a.cap_c2)
};

hipError_t launch_fwd16(const FwdArgs& a, bool is_bf16, FwdMode m, hipStream_t st);
// Local / soft-capped 16-bit launches (attn_fwd_local.hip).
hipError_t launch_fwd16_local(const FwdArgs& a, bool is_bf16, FwdMode m, hipStream_t st);
// Short key ranges with every key tile resident in LDS (attn_fwd_resident.hip):
// 16-bit, d <= 64, Nk <= kResidentMaxKeys, no mask / window / cap.
constexpr int kResidentMaxKeys = 224;
hipError_t launch_fwd16_resident(const FwdArgs& a, bool is_bf16, bool causal, hipStream_t st);
hipError_t launch_fwd32(const FwdArgs& a, FwdMode m, hipStream_t st);
// Backward launches take the forward's mode (mode.mask: a.mask is set).
hipError_t launch_bwd16(const BwdArgs& a, bool is_bf16, FwdMode m, hipStream_t st);
// fp32 backward (attn_bwd32.hip): D from dO and O, then dQ and dK/dV on the fp32 MFMA.
hipError_t launch_bwd32(const BwdArgs& a, FwdMode m, hipStream_t st);

}  // namespace attn
