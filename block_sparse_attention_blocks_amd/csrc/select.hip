// Block selector kernels for gfx950: block-mean pooling of Q and K, then
// per-row block scores and a deterministic top-k.
//
// The selector's contract is that of vllm-omni PR #8335 "[Core] Add shared
// block-sparse attention adapters with FlashAttention-4" (Purpose): it
// produces per-query-head KV-block indices and counts, always keeps the
// protected KV prefix, and query head h works against KV head h / G (native
// GQA mapping, K/V heads never repeated). The pages leave the scoring rule open; the
// reading implemented here is block-mean pooling of Q and K with the fp32 dot
// product of the pooled vectors as the block score, top-k by (score
// descending, index ascending).
//
// Exactness: the pooled vectors are the exact block sums (fp64 sums of bf16
// values) divided once in fp64 and rounded once to fp32; each score is the
// fp32 value nearest to the exact dot product of two pooled vectors. The fast
// path is an fp64 dot product with a rigorous error bound; when that bound
// leaves the fp32 rounding open, the score is recomputed with an exact
// 576-bit fixed-point accumulator. The selected set is therefore a pure
// function of the input bytes.

#include "internal.h"

namespace bsattn {
namespace {

// ---------------------------------------------------------------- pooling
// One workgroup of 512 threads per (batch, block, group of 2048 / D heads).
// The group's heads take A = heads x D / 8 threads, one 16-byte chunk of one
// head's row each; the S = min(512 / A, 8) thread sets split the block's
// rows among themselves (set s takes rows s, s + S, ...), and set 0 adds the
// other sets' partial sums through LDS. The rows are [rows][heads][D] bf16,
// so the reads stream; eight rows are in flight per thread. Sums are fp64
// and exact for these inputs, so the split changes no bit of the result.
constexpr int kPoolThreads = 512;

template <int D>
__global__ void __launch_bounds__(kPoolThreads) pool_kernel(const PoolParams p) {
  constexpr int CPH = D / 8;      // 16-byte chunks per head row
  constexpr int HPW = 256 / CPH;  // heads per workgroup
  __shared__ double part[kPoolThreads * 8];
  const int blk = blockIdx.x;
  const int b = blockIdx.z;
  const int h0 = blockIdx.y * HPW;
  const bool isq = blk < p.nq;
  const int j = isq ? blk : blk - p.nq;
  const int heads = isq ? p.hq : p.hkv;
  const int bs = isq ? p.bq : p.bk;
  const int start = j * bs;
  int end;
  if (isq) {
    end = min(start + bs, p.q_valid);
  } else {
    const int seg_end =
        (start < p.kv_prefix_len) ? p.kv_prefix_valid : p.kv_prefix_len + p.kv_suffix_valid;
    end = min(start + bs, seg_end);
  }
  const int n = max(end - start, 0);
  const uint16_t* base = isq ? p.q + (int64_t)b * p.qs0 : p.k + (int64_t)b * p.ks0;
  const int64_t s1 = isq ? p.qs1 : p.ks1;
  const int64_t s2 = isq ? p.qs2 : p.ks2;
  const int nblocks = isq ? p.nq : p.nk;
  if (h0 >= heads) return;  // the K blocks need fewer head groups than the Q blocks

  const int A = min(HPW, heads - h0) * CPH;  // threads per row set
  const int S = min(kPoolThreads / A, 8);    // row sets (set 0 adds the others one by one)
  const int c = (int)threadIdx.x;
  const int set = c / A, cc = c % A;
  const bool act = set < S;
  const int hh = h0 + cc / CPH;
  const int dc = cc % CPH;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  if (act) {
    const uint16_t* src = base + (int64_t)start * s1 + (int64_t)hh * s2 + dc * 8;
    // Eight rows per turn, all eight loads issued before the first is used;
    // rows past the block's real ones load nothing and add zeros (the sums
    // stay exact).
    for (int t0 = set; t0 < n; t0 += 8 * S) {
      uint4 raw[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int t = t0 + x * S;
        raw[x] = t < n ? *reinterpret_cast<const uint4*>(src + (int64_t)t * s1)
                       : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint32_t w[4] = {raw[x].x, raw[x].y, raw[x].z, raw[x].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)__uint_as_float(w[e] << 16);
          acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
    }
  }
  if (S > 1) {  // uniform over the workgroup
    if (act && set > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[e * kPoolThreads + c] = acc[e];
    }
    __syncthreads();
    if (set == 0) {
      for (int s = 1; s < S; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += part[e * kPoolThreads + s * A + cc];
    }
  }
  float m32[8];
  double sq = 0.0;
  const double dn = (double)max(n, 1);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m32[e] = n > 0 ? (float)(acc[e] / dn) : 0.0f;  // one fp64 division, one fp32 rounding
    sq = __builtin_fma((double)m32[e], (double)m32[e], sq);
  }
  // The CPH threads of one head row are consecutive lanes of one wave.
#pragma unroll
  for (int off = 1; off < CPH; off <<= 1) sq += __shfl_xor(sq, off);
  if (set == 0) {
    if (isq) {
      double* dst = p.qp + (((int64_t)b * p.hq + hh) * p.nq + j) * D + dc * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = (double)m32[e];
    } else {
      float* dst = p.kpt + (((int64_t)b * p.hkv + hh) * D + dc * 8) * p.nk + j;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[(int64_t)e * p.nk] = m32[e];
    }
    if (dc == 0) {
      // Upper bound of the Euclidean norm (covers the rounding of sq and sqrt).
      const double nrm = __builtin_sqrt(sq) * (1.0 + 0x1p-40);
      (isq ? p.qn : p.kn)[((int64_t)b * heads + hh) * nblocks + j] = nrm;
    }
  }
}

// ------------------------------------------------------- exact dot product
// Exact sum of D products of fp32 pairs in a 576-bit two's complement fixed
// point accumulator (bit 0 weighs 2^-298, below the smallest product
// 2^-149 * 2^-149; the largest sum stays below 2^561), then rounded to the
// nearest fp32, ties to even. A whole wave computes one sum: lane l adds the
// products l, l + 64, ... into its own accumulator, and a butterfly over the
// lanes adds the accumulators (additions modulo 2^576 are exact).
constexpr int kLimbs = 9;

// acc += the exact product of the fp32 values with bit patterns ua and ub.
__device__ __forceinline__ void acc_add_product(uint64_t (&acc)[kLimbs], uint32_t ua, uint32_t ub) {
  const uint32_t ea = (ua >> 23) & 0xFFu, eb = (ub >> 23) & 0xFFu;
  const uint64_t ma = (ua & 0x7FFFFFu) | (ea ? 0x800000u : 0u);
  const uint64_t mb = (ub & 0x7FFFFFu) | (eb ? 0x800000u : 0u);
  const uint64_t m = ma * mb;  // < 2^48
  if (m == 0) return;
  const int xa = ea ? (int)ea - 150 : -149;
  const int xb = eb ? (int)eb - 150 : -149;
  const int pos = xa + xb + 298;  // in [0, 506]
  const int limb = pos >> 6, off = pos & 63;
  const uint64_t lo = m << off;
  const uint64_t hi = off ? (m >> (64 - off)) : 0;
  const bool neg = ((ua ^ ub) >> 31) != 0;
  // acc += (neg ? -X : X), X = lo * 2^(64 limb) + hi * 2^(64 (limb + 1)); -X = ~X + 1.
  uint64_t carry = neg ? 1 : 0;
#pragma unroll
  for (int L = 0; L < kLimbs; ++L) {
    uint64_t x = (L == limb) ? lo : ((L == limb + 1) ? hi : 0);
    if (neg) x = ~x;
    const uint64_t s1 = acc[L] + x;
    const uint64_t c1 = s1 < x;
    const uint64_t s2 = s1 + carry;
    const uint64_t c2 = s2 < carry;
    acc[L] = s2;
    carry = c1 | c2;
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const int lo = __shfl_xor((int)(uint32_t)v, mask);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), mask);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Nearest fp32 (ties to even) of the fixed-point value.
__device__ __forceinline__ float acc_round_rn32(uint64_t (&acc)[kLimbs]) {
  const bool negr = (acc[kLimbs - 1] >> 63) != 0;
  if (negr) {  // magnitude
    uint64_t carry = 1;
#pragma unroll
    for (int L = 0; L < kLimbs; ++L) {
      const uint64_t x = ~acc[L];
      const uint64_t s = x + carry;
      carry = s < carry;
      acc[L] = s;
    }
  }
  int top = -1;  // highest set bit
#pragma unroll
  for (int L = kLimbs - 1; L >= 0; --L)
    if (top < 0 && acc[L] != 0) top = 64 * L + 63 - __clzll(acc[L]);
  if (top < 0) return 0.0f;  // exact zero: +0
  const int etop = top - 298;
  if (etop >= 128) return negr ? -__builtin_inff() : __builtin_inff();
  const int lsb = (etop >= -126) ? top - 23 : 149;  // weight 2^(lsb-298) of the last kept bit
  const int sbit = lsb - 1;                          // round bit, >= 148
  const int wl = sbit >> 6, wo = sbit & 63;
  uint64_t w0 = 0, w1 = 0;
  bool sticky = false;
#pragma unroll
  for (int L = 0; L < kLimbs; ++L) {
    if (L == wl) {
      w0 = acc[L];
      sticky = sticky || (wo ? (acc[L] & ((1ull << wo) - 1)) != 0 : false);
    }
    if (L == wl + 1) w1 = acc[L];
    if (L < wl) sticky = sticky || acc[L] != 0;
  }
  const uint64_t win = (w0 >> wo) | (wo ? (w1 << (64 - wo)) : 0);
  const bool round = (win & 1) != 0;
  uint64_t mant = (win >> 1) & 0xFFFFFFull;
  if (round && (sticky || (mant & 1))) mant += 1;
  const float mag = (float)__builtin_ldexp((double)mant, lsb - 298);  // exact in fp32
  return negr ? -mag : mag;
}

// a: D values (fp32 held exactly in fp64), b: D fp32 values at stride
// bstride. Called by a whole wave with uniform arguments; every lane returns
// the result.
__device__ __noinline__ float exact_dot_rn32_wave(const double* a, const float* b, int64_t bstride,
                                                  int D, int lane) {
  uint64_t acc[kLimbs];
#pragma unroll
  for (int L = 0; L < kLimbs; ++L) acc[L] = 0;
  for (int d = lane; d < D; d += 64)
    acc_add_product(acc, __float_as_uint((float)a[d]), __float_as_uint(b[(int64_t)d * bstride]));
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    uint64_t carry = 0;
#pragma unroll
    for (int L = 0; L < kLimbs; ++L) {
      const uint64_t x = shfl_xor_u64(acc[L], sh);
      const uint64_t s1 = acc[L] + x;
      const uint64_t c1 = s1 < x;
      const uint64_t s2 = s1 + carry;
      const uint64_t c2 = s2 < carry;
      acc[L] = s2;
      carry = c1 | c2;
    }
  }
  return acc_round_rn32(acc);
}

// Minimum over the wave's 64 lanes (every lane gets it).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, sh));
  return v;
}

// Key of a score whose fp32 rounding the fp64 bound leaves open; above every
// key of a finite score.
constexpr uint32_t kUndecided = 0xFFFFFFFFu;

// Monotone map of fp32 values to unsigned keys (-0 and +0 map alike).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------ scores and top-k
// Workgroup = R consecutive query blocks of one (batch, query head). Phase 1:
// the block scores of a 16-row x 16-candidate tile come from the fp64 matrix
// cores (v_mfma_f64_16x16x4_f64, 4 head-dim entries per step): A (16 x 4)
// holds the pooled query rows, lane l carrying row l % 16, entry l / 16; B
// (4 x 16) the pooled keys, lane l carrying candidate l % 16, entry l / 16;
// entry e of the result in lane l is row 4 e + l / 16, candidate l % 16.
// Every product of two fp32 values is exact in fp64 and each accumulation is
// rounded once, so the rigorous error bound of an fp64 dot product applies.
// Phase 2: each wave takes rows and selects the top blocks by bisection on
// the 32-bit keys, then writes the list in ascending block order. NW waves
// share both phases: eight, or sixteen when the grid has fewer workgroups
// than the chip has CUs (few heads), where a workgroup's latency is the
// call's time.
template <int D, int R, int NW>
__global__ void __launch_bounds__(64 * NW) score_topk_kernel(const ScoreParams p) {
  extern __shared__ uint32_t keys_lds[];
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  constexpr int KST = D / 4;  // MFMA k-steps over D
  const int ncand = p.n_cand;
  const int ncp = (ncand + 63) & ~63;
  const int i0 = blockIdx.x * R;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrows = min(R, p.nq - i0);
  const double* __restrict__ qrows = p.qp + (((int64_t)b * p.hq + h) * p.nq + i0) * D;
  const double* __restrict__ qnorm = p.qn + ((int64_t)b * p.hq + h) * p.nq + i0;
  const float* __restrict__ kcols = p.kpt + ((int64_t)b * p.hkv + g) * D * (int64_t)p.nk;
  const double* __restrict__ knorm = p.kn + ((int64_t)b * p.hkv + g) * p.nk;
  const double gamma2 = 2.0 * (double)(D + 2) * 0x1p-53;

  const int arow = lane & 15, kq = lane >> 4;
  double qa[KST];
  {
    const double* qr = qrows + (int64_t)min(arow, nrows - 1) * D + kq;
#pragma unroll
    for (int st = 0; st < KST; ++st) qa[st] = qr[4 * st];
  }
  const int ntiles = (ncand + 15) >> 4;
  for (int tile = wave; tile < ntiles; tile += NW) {
    const int c = tile * 16 + arow;  // candidate of this lane (B column, result column)
    const int j = p.n_prefix_blocks + min(c, ncand - 1);
    const float* kc = kcols + j + (int64_t)kq * p.nk;
    float kb[KST];
#pragma unroll
    for (int st = 0; st < KST; ++st) kb[st] = kc[(int64_t)(4 * st) * p.nk];
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int st = 0; st < KST; ++st)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[st], (double)kb[st], acc, 0, 0, 0);
    if (c < ncand) {
      const double knj = knorm[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * e + kq;
        if (r < nrows) {
          const double sc = acc[e];
          const double w = gamma2 * qnorm[r] * knj + __builtin_fabs(sc) * 0x1p-52;
          const float lo = (float)(sc - w);
          const float hi = (float)(sc + w);
          // Undecided roundings are marked and recomputed exactly below, out
          // of this loop (finite scores never map to the marker).
          keys_lds[r * ncp + c] =
              __float_as_uint(lo) != __float_as_uint(hi) ? kUndecided : order_key(lo);
        }
      }
    }
  }
  __syncthreads();
  // Exact recomputation of the marked scores (rare: a few in a hundred
  // thousand for typical inputs, but any number is handled), one whole wave
  // per score.
  for (int e0 = wave * 64; e0 < nrows * ncp; e0 += 64 * NW) {
    const int e = e0 + lane;
    // Slots past the row's candidates (c >= ncand) were never written.
    uint64_t marked = __builtin_amdgcn_ballot_w64(e < nrows * ncp && (e % ncp) < ncand &&
                                                  keys_lds[e] == kUndecided);
    while (marked != 0) {
      const int ee = e0 + (int)__builtin_ctzll(marked);
      marked &= marked - 1;
      const int r = ee / ncp, c = ee % ncp;
      const float f = exact_dot_rn32_wave(qrows + (int64_t)r * D, kcols + p.n_prefix_blocks + c,
                                          p.nk, D, lane);
      if (lane == 0) keys_lds[ee] = order_key(f);
    }
  }
  __syncthreads();

  const int rsel = min(p.keep - p.n_forced, ncand);
  const bool take_all = rsel == ncand;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int M = ncp >> 6;
  for (int r = wave; r < nrows; r += NW) {
    const int i = i0 + r;
    const int64_t row_id = ((int64_t)b * p.hq + h) * p.nq + i;
    int32_t* out = p.idx + row_id * p.idx_row_stride;
    const bool row_ok = (int64_t)i * p.bq < (int64_t)p.q_valid;
    int written = 0;
    if (row_ok) {
      const uint32_t* kr = keys_lds + r * ncp;
      uint32_t thr = 0;
      int need_eq = 0;
      if (rsel > 0 && !take_all) {
        // Largest thr with #{key >= thr} >= rsel: the rsel-th largest key.
        // Every real key is at least order_key(-inf) > 0, so the 0 standing
        // in for a missing candidate never counts.
        if constexpr (R == 16) {
          // At most 1024 candidates: the row's keys stay in registers.
          uint32_t kreg[16];
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const int jj = m * 64 + lane;
            kreg[m] = (m < M && jj < ncand) ? kr[jj] : 0u;
          }
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int count = 0;
#pragma unroll
            for (int m = 0; m < 16; ++m)
              if (m < M) count += __popcll(__ballot(kreg[m] >= cand));
            if (count == rsel) {
              // Exactly the rsel largest keys are >= cand: the threshold is
              // the smallest of them.
              uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
              for (int m = 0; m < 16; ++m)
                if (m < M && kreg[m] >= cand) mn = min(mn, kreg[m]);
              thr = wave_min_u32(mn);
              break;
            }
            if (count > rsel) thr = cand;
          }
          int gt = 0;
#pragma unroll
          for (int m = 0; m < 16; ++m)
            if (m < M) gt += __popcll(__ballot(kreg[m] > thr));
          need_eq = rsel - gt;  // >= 1
        } else {
          for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = thr | (1u << bit);
            int count = 0;
            for (int m = 0; m < M; ++m) {
              const int jj = m * 64 + lane;
              count += __popcll(__ballot(jj < ncand && kr[jj] >= cand));
            }
            if (count == rsel) {
              uint32_t mn = 0xFFFFFFFFu;
              for (int m = 0; m < M; ++m) {
                const int jj = m * 64 + lane;
                if (jj < ncand && kr[jj] >= cand) mn = min(mn, kr[jj]);
              }
              thr = wave_min_u32(mn);
              break;
            }
            if (count > rsel) thr = cand;
          }
          int gt = 0;
          for (int m = 0; m < M; ++m) {
            const int jj = m * 64 + lane;
            gt += __popcll(__ballot(jj < ncand && kr[jj] > thr));
          }
          need_eq = rsel - gt;  // >= 1
        }
      }
      for (int s = lane; s < p.n_forced; s += 64) out[s] = s;
      int pos = p.n_forced;
      if (rsel > 0) {
        int eq_seen = 0;
        for (int m = 0; m < M; ++m) {
          const int jj = m * 64 + lane;
          const bool in = jj < ncand;
          const uint32_t key = in ? kr[jj] : 0u;
          const bool gt = in && (take_all || key > thr);
          const bool eq = in && !take_all && key == thr;
          const uint64_t eqm = __ballot(eq);
          const int eq_before = eq_seen + __popcll(eqm & lt_mask);
          const bool sel = gt || (eq && eq_before < need_eq);
          const uint64_t selm = __ballot(sel);
          const int slot = pos + __popcll(selm & lt_mask);
          if (sel && slot < p.idx_row_stride) out[slot] = p.n_prefix_blocks + jj;
          pos += __popcll(selm);
          eq_seen += __popcll(eqm);
        }
      }
      written = pos;
    }
    for (int s = written + lane; s < p.idx_row_stride; s += 64) out[s] = -1;
    if (lane == 0) p.cnt[row_id] = written;
  }
}

}  // namespace

int score_rows_per_wg(int n_cand) { return n_cand <= 1024 ? 16 : 8; }

size_t score_lds_bytes(int n_cand) {
  const size_t ncp = (size_t)((n_cand + 63) & ~63);
  return (size_t)score_rows_per_wg(n_cand) * ncp * sizeof(uint32_t);
}

hipError_t launch_pool(const PoolParams& p, int head_dim, int batch, hipStream_t stream) {
  const int hpw = 256 / (head_dim / 8);
  const int hmax = p.hq > p.hkv ? p.hq : p.hkv;
  const dim3 grid(p.nq + p.nk, (hmax + hpw - 1) / hpw, batch);
  if (grid.x == 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(kPoolThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(kPoolThreads), 0, stream, p);
  return hipGetLastError();
}

namespace {

template <int D, int R, int NW>
hipError_t launch_score_one(const ScoreParams& p, dim3 grid, size_t lds, hipStream_t stream) {
  // Kernels taking more than 64 KiB of dynamic LDS must say so first.
  static const hipError_t attr_status = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&score_topk_kernel<D, R, NW>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr_status != hipSuccess) return attr_status;
  hipLaunchKernelGGL((score_topk_kernel<D, R, NW>), grid, dim3(64 * NW), lds, stream, p);
  return hipGetLastError();
}

template <int D, int R>
hipError_t launch_score_waves(const ScoreParams& p, dim3 grid, size_t lds, hipStream_t stream) {
  const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
  return wgs < 256 ? launch_score_one<D, R, 16>(p, grid, lds, stream)
                   : launch_score_one<D, R, 8>(p, grid, lds, stream);
}

}  // namespace

hipError_t launch_score_topk(const ScoreParams& p, int head_dim, int batch, hipStream_t stream) {
  const int rows = score_rows_per_wg(p.n_cand);
  const dim3 grid((p.nq + rows - 1) / rows, p.hq, batch);
  if (grid.x == 0) return hipSuccess;
  const size_t lds = score_lds_bytes(p.n_cand);
  if (head_dim == 128)
    return rows == 16 ? launch_score_waves<128, 16>(p, grid, lds, stream)
                      : launch_score_waves<128, 8>(p, grid, lds, stream);
  return rows == 16 ? launch_score_waves<64, 16>(p, grid, lds, stream)
                    : launch_score_waves<64, 8>(p, grid, lds, stream);
}

}  // namespace bsattn
