// Selected-block attention forward kernel for gfx950 (CDNA4).
//
// What it computes (vllm-omni PR #8335 "[Core] Add shared block-sparse
// attention adapters with FlashAttention-4", Purpose; diffusers
// examples/cosmos3/cosmos_parallel.py, cosmos3_cp_attention and
// build_gen_key_mask): for every query row of a query block, non-causal
// softmax attention over the keys of the KV blocks listed for that
// (batch, query head, query block), padded keys excluded, query head h
// reading KV head h / G in place. The dense case is the same kernel with the
// list "every non-empty block" generated in-kernel.
//
// Structure (one workgroup per query block, one wave per 32 query rows):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the K tile (A operand) comes
//    from LDS, Q^T (B operand) stays in registers for the whole row block.
//    Each lane then owns one query row (lane % 32) and half of the tile's
//    keys, so the row max / row sum need a single cross-lane step.
//  * Online softmax in fp32, exp2 with the scale folded into one FMA.
//  * O^T = V^T P^T with the same MFMA: P^T is the S^T accumulator converted
//    to bf16 in place (the contraction over keys is order-free, so the key
//    order of the accumulator layout is reused for V); V^T fragments are
//    read from the row-major V tile with ds_read_b64_tr_b16. The output
//    accumulator again has one query per lane, so the softmax rescale is a
//    per-lane multiply.
//  * K and V tiles move HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), XOR-swizzled in 16-byte chunks so the K row reads and the
//    V transpose reads hit distinct banks. K of the next block loads while
//    this block's softmax and PV run; V of the next block loads while the
//    next QK^T and softmax run.
//  * Workgroups are renumbered so that each XCD works through a contiguous
//    range of (KV head, query block), keeping that range's K/V tiles in the
//    XCD's L2.

#include "internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Chunk permutation of row `row` in an LDS tile with CPR 16-byte chunks.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  return ((row & 7) << 1) & (CPR - 1);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Issue the HBM->LDS copy of one [BK x D] bf16 tile. `src` points at row 0 of
// the tile for the right batch and KV head; rows are `row_stride` elements
// apart. Each wave instruction moves 64 x 16 bytes = RPI whole rows.
template <int D, int BK, int NW>
__device__ __forceinline__ void issue_tile(const uint16_t* src, int64_t row_stride, uint16_t* lds,
                                           int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int NL = BK / (NW * RPI);
  static_assert(NL * NW * RPI == BK, "tile split");
  const int rsub = lane / CPR;
  const int pch = lane % CPR;
#pragma unroll
  for (int it = 0; it < NL; ++it) {
    const int rbase = (it * NW + wave) * RPI;
    const int row = rbase + rsub;
    const int lch = pch ^ swz<CPR>(row);
    const uint16_t* g = src + (int64_t)row * row_stride + lch * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)(lds + rbase * D),
                                     16, 0, 0);
  }
}

template <int D, int BQ, int BK, bool DENSE>
__global__ void __launch_bounds__(BQ * 2) __attribute__((amdgpu_waves_per_eu(2)))
attn_fwd_kernel(const AttnParams p) {
  constexpr int NW = BQ / 32;
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int NL = BK / (NW * RPI);  // copy instructions per thread per tile
  constexpr int KS = D / 16;           // MFMA k-steps over D
  constexpr int DT = D / 32;           // output 32-row tiles over D
  constexpr int KT = BK / 32;          // 32-key sub-tiles per block
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BK * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BK * D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;

  // Workgroup w runs on XCD w % 8; give each XCD a contiguous range of the
  // (batch, KV head, query block, head-in-group) order.
  const int nwg = p.n_wg;
  const int w = blockIdx.x;
  const int xcd = w & 7, per = nwg >> 3, rem = nwg & 7;
  const int lin = xcd * per + min(xcd, rem) + (w >> 3);
  const int hig = lin % p.group;
  int t = lin / p.group;
  const int i = t % p.nq;
  t /= p.nq;
  const int g = t % p.hkv;
  const int b = t / p.hkv;
  const int h = g * p.group + hig;

  const int row0 = i * BQ;
  const int qrow = row0 + wave * 32 + col;

  // Q^T fragments (B operand): lane holds q[qrow][16 ks + 8 half .. +7].
  bf16x8 qf[KS];
  {
    const uint16_t* qp = p.q + (int64_t)b * p.qs0 + (int64_t)qrow * p.qs1 + (int64_t)h * p.qs2 +
                         half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  int nblk;
  const int32_t* idx_row = nullptr;
  if constexpr (DENSE) {
    nblk = p.n_forced + p.n_cand;
  } else {
    const int64_t row_id = ((int64_t)b * p.hq + h) * p.nq + i;
    nblk = min(max(p.cnt[row_id], 0), p.idx_row_stride);
    idx_row = p.idx + row_id * p.idx_row_stride;
  }
  if (row0 >= p.q_valid) nblk = 0;

  const uint16_t* kbase = p.k + (int64_t)b * p.ks0 + (int64_t)g * p.ks2;
  const uint16_t* vbase = p.v + (int64_t)b * p.vs0 + (int64_t)g * p.vs2;

  auto block_of = [&](int n) -> int {
    if constexpr (DENSE) {
      return n < p.n_forced ? n : p.n_prefix_blocks + (n - p.n_forced);
    } else {
      return idx_row[n];
    }
  };
  // Real keys of block j form a prefix [0, nvalid) of the block: segments
  // are block aligned and padding follows the real keys of each segment.
  auto nvalid_of = [&](int j) -> int {
    if (j < 0 || j >= p.nk) return 0;
    const int s0 = j * BK;
    const int seg_end =
        (s0 < p.kv_prefix_len) ? p.kv_prefix_valid : p.kv_prefix_len + p.kv_suffix_valid;
    return min(max(seg_end - s0, 0), BK);
  };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  const float sl2 = p.scale_log2;

  // LDS read offsets that do not depend on the block.
  const int g16 = lane >> 4, j16 = lane & 15, tq = j16 >> 2, q4 = j16 & 3;

  int j_cur = -1, nv_cur = 0;
  if (nblk > 0) {
    j_cur = block_of(0);
    nv_cur = nvalid_of(j_cur);
    if (nv_cur > 0) {
      issue_tile<D, BK, NW>(kbase + (int64_t)j_cur * BK * p.ks1, p.ks1, Ks, wave, lane);
      issue_tile<D, BK, NW>(vbase + (int64_t)j_cur * BK * p.vs1, p.vs1, Vs, wave, lane);
    }
  }

  for (int n = 0; n < nblk; ++n) {
    int j_nxt = -1, nv_nxt = 0;
    if (n + 1 < nblk) {
      j_nxt = block_of(n + 1);
      nv_nxt = nvalid_of(j_nxt);
    }
    f32x16 s[KT];
    if (nv_cur > 0) {
      wait_vmcnt<NL>();  // K of this block has landed (its V may still be in flight)
      __syncthreads();
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
        const int row = kt * 32 + col;
        const uint16_t* krow = Ks + row * D;
        const int sw = swz<CPR>(row);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = (2 * ks + half) ^ sw;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ch * 8);
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // every wave is done with the K tile
    if (nv_nxt > 0)
      issue_tile<D, BK, NW>(kbase + (int64_t)j_nxt * BK * p.ks1, p.ks1, Ks, wave, lane);

    if (nv_cur > 0) {
      // ---- online softmax on S^T: lane owns query col, keys
      //      kt*32 + (r/4)*8 + half*4 + r%4.
      if (nv_cur < BK) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            if (key >= nv_cur) s[kt][r] = -__builtin_inff();
          }
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kt][r]);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = __builtin_fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == -__builtin_inff()) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float rs = 0.0f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], sl2, -m_use));
          s[kt][r] = e;
          rs += e;
        }
      rs += __shfl_xor(rs, 32);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

      // P^T as the B operand: k-step (kt, s2) takes accumulator entries
      // r = 8 s2 .. 8 s2 + 7, i.e. keys kt*32 + 16 s2 + {4 half + 0..3, 8 + 4 half + 0..3}.
      bf16x8 pf[2 * KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[2 * kt + s2][e] = (__bf16)s[kt][8 * s2 + e];

      if (nv_nxt > 0)
        wait_vmcnt<NL>();  // V of this block has landed (next K may be in flight)
      else
        wait_vmcnt<0>();
      __syncthreads();
      if (nv_cur < BK) {
        // Padded keys get weight 0, but 0 * NaN is NaN: clear their V rows.
        constexpr int NT = NW * 64;
        uint4* vz = reinterpret_cast<uint4*>(Vs + nv_cur * D);
        const int nz = (BK - nv_cur) * D / 8;
        for (int e = threadIdx.x; e < nz; e += NT) vz[e] = make_uint4(0, 0, 0, 0);
        __syncthreads();
      }

      // ---- O^T += V^T P^T. V^T fragment of lane: row d = dt*32 + col,
      //      k-slots 0..3 / 4..7 = keys base + 0..3 / base + 8 + 0..3 with
      //      base = kt*32 + 16 s2 + 4 half; one transpose read per group of 4.
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            bf16x4 v0, v1;
            const int d = dt * 32 + 16 * (g16 & 1) + 4 * q4;
            {
              const int row = kt * 32 + 16 * s2 + 4 * half + tq;
              const int off = row * D + (((d >> 3) ^ swz<CPR>(row)) << 3) + (d & 7);
              v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vs + off));
            }
            {
              const int row = kt * 32 + 16 * s2 + 8 + 4 * half + tq;
              const int off = row * D + (((d >> 3) ^ swz<CPR>(row)) << 3) + (d & 7);
              v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Vs + off));
            }
            const bf16x8 a = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[2 * kt + s2], o[dt], 0, 0, 0);
          }
        }
    }
    __syncthreads();  // every wave is done with the V tile
    if (nv_nxt > 0)
      issue_tile<D, BK, NW>(vbase + (int64_t)j_nxt * BK * p.vs1, p.vs1, Vs, wave, lane);
    j_cur = j_nxt;
    nv_cur = nv_nxt;
  }

  // ---- epilogue: O^T lane layout is query col, d = dt*32 + (r/4)*8 + half*4 + r%4.
  const bool row_ok = qrow < p.q_valid && l_run > 0.0f;
  const float inv = row_ok ? 1.0f / l_run : 0.0f;
  uint16_t* op = p.o + (int64_t)b * p.os0 + (int64_t)qrow * p.os1 + (int64_t)h * p.os2;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      bf16x4 vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = (__bf16)(row_ok ? o[dt][rg * 4 + e] * inv : 0.0f);
      *reinterpret_cast<bf16x4*>(op + dt * 32 + rg * 8 + half * 4) = vv;
    }
  if (p.lse != nullptr && half == 0) {
    const float lse = row_ok ? (m_run + __builtin_log2f(l_run)) * 0.69314718055994531f
                             : -__builtin_inff();
    p.lse[((int64_t)b * p.hq + h) * p.q_len + qrow] = lse;
  }
}

template <int D, int BQ, int BK, bool DENSE>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, BQ, BK, DENSE>), dim3(p.n_wg), dim3(BQ * 2), 0, stream,
                     p);
  return hipGetLastError();
}

template <int D, int BQ, int BK>
hipError_t launch_mode(const AttnParams& p, bool dense, hipStream_t stream) {
  return dense ? launch_one<D, BQ, BK, true>(p, stream) : launch_one<D, BQ, BK, false>(p, stream);
}

template <int D>
hipError_t launch_geom(const AttnParams& p, int bq, int bk, bool dense, hipStream_t stream) {
  if (bq == 64 && bk == 64) return launch_mode<D, 64, 64>(p, dense, stream);
  if (bq == 64 && bk == 128) return launch_mode<D, 64, 128>(p, dense, stream);
  if (bq == 128 && bk == 64) return launch_mode<D, 128, 64>(p, dense, stream);
  return launch_mode<D, 128, 128>(p, dense, stream);
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int head_dim, int block_q, int block_k, bool dense,
                            hipStream_t stream) {
  if (p.n_wg == 0) return hipSuccess;
  if (head_dim == 128) return launch_geom<128>(p, block_q, block_k, dense, stream);
  return launch_geom<64>(p, block_q, block_k, dense, stream);
}

}  // namespace bsattn
