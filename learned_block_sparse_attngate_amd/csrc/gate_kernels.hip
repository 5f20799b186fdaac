// AttnGate for gfx950: block pooling, per-head projections, block-level RoPE,
// causal block-level softmax and the threshold / top-k block mask; the
// gate's self-distillation step; and the decode-stage gate (compressed K
// cache, per-token scores and mask).
//
// Method ("SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
// explainer section 3.4, "AttnGate" and its score equation, "Pooling Method
// Selection", "Inference Procedure" Methods 1 and 2; "SeerAttention:
// Self-distilled Attention Gating for Efficient Long-context Prefilling",
// response 3.3 on mask generation):
//   Qp = AvgPool_64(Q), Kp = [MaxPool_64 | MinPool_64 | AvgPool_64](K),
//   score = softmax_row((Qp W_q)(Kp W_k)^T / sqrt(d)) over key blocks j <= i,
//   mask = score > T, or the top-k entries of each row.
//
// Everything stays in fp32 so that the mask, which is a hard decision on the
// scores, is reproducible against an fp64 reference except for scores within
// rounding distance of the threshold.
//
// Kernels:
//  gate_pool        HBM-bound: one workgroup per (head, block) streams the 64
//                   token rows once with 16-byte loads and reduces in LDS.
//  gate_gemm        fp32 LDS-tiled GEMM on the fp32 matrix cores (64 x 64
//                   tiles, a 32 x 32 quadrant per wavefront), used for the
//                   two projections, the causal tiles of the block logits
//                   Q' K'^T and the distillation step's gradients.
//  gate_softmax_mask_wave
//                   one wavefront per score row (rows up to 4096 blocks), the
//                   row in registers: max / sum reductions, the normalized
//                   row, and either the threshold or the exact k-th largest
//                   for top-k (exponent by ballot counts, mantissa by radix
//                   passes; ties to the lower index).
//  gate_softmax_mask the same with one workgroup per row, for longer rows.
//  gate_rope        in-place block-level RoPE of Q' / K' (fp64 angles).
//  gate_kl, gate_dproj, gate_dweight, gate_loss
//                   the distillation step: KL rows and dz, dQ' / dK' GEMMs,
//                   weight-gradient GEMMs, fixed-order loss reduction.
//  decode_kcomp, decode_logits, decode_gate
//                   decode stage: pooled and projected key blocks, 8 lanes
//                   per logit, then the row softmax and mask (a workgroup per
//                   row: with one row per head, four wavefronts per row hide
//                   more latency than one).
#include <math.h>

#include "seer_device.h"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kPoolThreads = 256;

// block i of head row y (b * (Hq + Hkv) + query head, or + Hq + KV head)
template <int D>
__device__ __forceinline__ void gate_pool_body(const GateArgs& a, const int i, const int y) {
  constexpr int CPR = D / 8;              // 16-byte chunks per token row
  constexpr int NRG = kPoolThreads / CPR; // row groups
  __shared__ float red[3][NRG][D];

  const int H = a.Hq + a.Hkv;
  const int b = y / H;
  const int hx = y - b * H;
  const bool isq = hx < a.Hq;
  const uint16_t* src = isq ? a.q + (static_cast<size_t>(b) * a.Hq + hx) * a.hs * D
                            : a.k + (static_cast<size_t>(b) * a.Hkv + (hx - a.Hq)) * a.hs * D;
  const int t0 = i * kBlock;
  const int n = min(kBlock, a.S - t0);
  const int tid = threadIdx.x;
  const int c = tid % CPR;
  const int rg = tid / CPR;

  float sum[8], mx[8], mn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { sum[e] = 0.f; mx[e] = -INFINITY; mn[e] = INFINITY; }
  // all of the thread's rows are loaded before any is reduced (one memory
  // round trip per workgroup); rows past a ragged last block re-read the
  // block's last row and are skipped below
  constexpr int RPT = kBlock / NRG;       // rows per thread
  uint4 rows[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = min(rg + u * NRG, n - 1);
    rows[u] = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(t0 + r) * D + 8 * c);
  }
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    if (rg + u * NRG >= n) continue;
    const uint32_t w[4] = {rows[u].x, rows[u].y, rows[u].z, rows[u].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
      sum[e] += x;
      mx[e] = fmaxf(mx[e], x);
      mn[e] = fminf(mn[e], x);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][rg][8 * c + e] = sum[e];
    red[1][rg][8 * c + e] = mx[e];
    red[2][rg][8 * c + e] = mn[e];
  }
  __syncthreads();
  const float inv_n = 1.0f / static_cast<float>(n);
  for (int d = tid; d < D; d += kPoolThreads) {
    float s = 0.f, hi = -INFINITY, lo = INFINITY;
    for (int r = 0; r < NRG; ++r) {
      s += red[0][r][d];
      hi = fmaxf(hi, red[1][r][d]);
      lo = fminf(lo, red[2][r][d]);
    }
    if (isq) {
      a.qp[((static_cast<size_t>(b) * a.Hq + hx) * a.nb + i) * D + d] = s * inv_n;
    } else {
      float* o = a.kp + ((static_cast<size_t>(b) * a.Hkv + (hx - a.Hq)) * a.nb + i) * (3 * D);
      o[d] = hi;
      o[D + d] = lo;
      o[2 * D + d] = s * inv_n;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kPoolThreads) void gate_pool_kernel(GateArgs a) {
  gate_pool_body<D>(a, blockIdx.x, blockIdx.y);
}

// ---------------------------------------------------------------------------
// fp32 tiled GEMM: C[m][n] = alpha * sum_k A[m][k] * Bm(k, n)
//   Bm(k, n) = B[k*ldb + n] (B_T = false) or B[n*ldb + k] (B_T = true)
// ---------------------------------------------------------------------------
constexpr int kGT = 256;
constexpr int kBM = 64, kBN = 64, kBK = 16;
static_assert(kBM == kGateTile, "the host builds varlen tile prefixes with kGateTile");

// acc += A(m0 .. m0+63, k) * Bm(k, n0 .. n0+63) over k in [k0, k1), where
// A(m, k) = A[m*lda + k] (A_T = false) or A[k*lda + m] (A_T = true), on the
// fp32 matrix cores: wave w owns the 32 x 32 quadrant at rows 32 (w & 1),
// columns 32 (w >> 1), and lane l's element r is its entry
// [8 (r / 4) + 4 (l / 32) + r % 4][l % 32] (v_mfma_f32_32x32x2_f32: lane l
// supplies A[l % 32][l / 32] and B[l / 32][l % 32] of each 32 x 2 x 32 step).
template <bool A_T, bool B_T>
__device__ __forceinline__ void gemm_accum(f32x16_t& acc, const float* __restrict__ A, int lda,
                                           const float* __restrict__ B, int ldb, int M, int N, int k0, int k1,
                                           int m0, int n0) {
  __shared__ __align__(16) float As[kBK][kBM + 4];
  __shared__ __align__(16) float Bs[kBK][kBN + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int qm = 32 * (w & 1) + (lane & 31), qn = 32 * (w >> 1) + (lane & 31), kh = lane >> 5;
  // 16-byte loads (one per operand and thread) for chunks inside the matrices
  // when the strides and bases allow them; 4-byte loads otherwise
  const bool vec_ok = (((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15) == 0) &&
                      ((lda | ldb | k0) & 3) == 0 && m0 + kBM <= M && n0 + kBN <= N;
  // the next chunk's operands are loaded into registers while this chunk's
  // products run: A tile 64 x 16 (stored transposed), B tile 16 x 64
  float ra[4], rb[4];
  bool rvec = false;                         // ra / rb hold one 16-byte group each
  // 16-byte group of thread t: A (m, k..k+3) or, transposed, (k, m..m+3);
  // B (k, n..n+3) or, transposed, (n, k..k+3)
  const int va_r = A_T ? (tid >> 4) : (tid >> 2), va_c = A_T ? 4 * (tid & 15) : 4 * (tid & 3);
  const int vb_r = B_T ? (tid >> 2) : (tid >> 4), vb_c = B_T ? 4 * (tid & 3) : 4 * (tid & 15);
  auto gload = [&](int kb) {
    rvec = vec_ok && kb + kBK <= k1;
    if (rvec) {
      const float4 x = A_T ? *reinterpret_cast<const float4*>(A + static_cast<size_t>(kb + va_r) * lda + m0 + va_c)
                           : *reinterpret_cast<const float4*>(A + static_cast<size_t>(m0 + va_r) * lda + kb + va_c);
      const float4 y = B_T ? *reinterpret_cast<const float4*>(B + static_cast<size_t>(n0 + vb_r) * ldb + kb + vb_c)
                           : *reinterpret_cast<const float4*>(B + static_cast<size_t>(kb + vb_r) * ldb + n0 + vb_c);
      ra[0] = x.x; ra[1] = x.y; ra[2] = x.z; ra[3] = x.w;
      rb[0] = y.x; rb[1] = y.y; rb[2] = y.z; rb[3] = y.w;
      return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + kGT * e;         // 0..1023
      const int am = A_T ? (idx & 63) : (idx >> 4), ak = A_T ? (idx >> 6) : (idx & 15);
      const int gm = m0 + am, gk = kb + ak;
      ra[e] = 0.f;
      if (gm < M && gk < k1) ra[e] = A_T ? A[static_cast<size_t>(gk) * lda + gm] : A[static_cast<size_t>(gm) * lda + gk];
      const int bn = B_T ? (idx >> 4) : (idx & 63), bk = B_T ? (idx & 15) : (idx >> 6);
      const int gn = n0 + bn, gk2 = kb + bk;
      rb[e] = 0.f;
      if (gn < N && gk2 < k1) rb[e] = B_T ? B[static_cast<size_t>(gn) * ldb + gk2] : B[static_cast<size_t>(gk2) * ldb + gn];
    }
  };
  if (k0 < k1) gload(k0);
  for (int kb = k0; kb < k1; kb += kBK) {
    if (rvec) {
      if (A_T) {
        *reinterpret_cast<float4*>(&As[va_r][va_c]) = make_float4(ra[0], ra[1], ra[2], ra[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) As[va_c + e][va_r] = ra[e];
      }
      if (B_T) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[vb_c + e][vb_r] = rb[e];
      } else {
        *reinterpret_cast<float4*>(&Bs[vb_r][vb_c]) = make_float4(rb[0], rb[1], rb[2], rb[3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = tid + kGT * e;
        As[A_T ? (idx >> 6) : (idx & 15)][A_T ? (idx & 63) : (idx >> 4)] = ra[e];
        Bs[B_T ? (idx & 15) : (idx >> 6)][B_T ? (idx >> 4) : (idx & 63)] = rb[e];
      }
    }
    __syncthreads();
    if (kb + kBK < k1) gload(kb + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[kk + kh][qm], Bs[kk + kh][qn], acc, 0, 0, 0);
    __syncthreads();
  }
}

__device__ __forceinline__ void gemm_store(const f32x16_t& acc, float* __restrict__ C, int ldc, int M, int N,
                                           int m0, int n0, float alpha, bool causal_only) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int gn = n0 + 32 * (w >> 1) + (lane & 31);
  if (gn >= N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int gm = m0 + 32 * (w & 1) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (gm >= M || (causal_only && gn > gm)) continue;
    C[static_cast<size_t>(gm) * ldc + gn] = acc[r] * alpha;
  }
}

// C = alpha * A Bm over the full K (one 64 x 64 tile)
template <bool B_T>
__device__ __forceinline__ void gemm_tile(const float* __restrict__ A, int lda, const float* __restrict__ B,
                                          int ldb, float* __restrict__ C, int ldc, int M, int N, int K,
                                          int m0, int n0, float alpha, bool causal_only) {
  f32x16_t acc = {};
  gemm_accum<false, B_T>(acc, A, lda, B, ldb, M, N, 0, K, m0, n0);
  gemm_store(acc, C, ldc, M, N, m0, n0, alpha, causal_only);
}

// Projections. blockIdx.z: 0 .. B*Hq-1 are Q' (one per query head), the rest
// are K' (one per query head, or one per KV head).
__device__ __forceinline__ void gate_proj_body(const GateArgs& a, const int bx, const int by, const int z) {
  const int nq = a.B * a.Hq;
  const int m0 = bx * kBM, n0 = by * kBN;
  if (z < nq) {
    const int h = z % a.Hq;
    gemm_tile<false>(a.qp + static_cast<size_t>(z) * a.nb * a.D, a.D, a.wq + static_cast<size_t>(h) * a.D * a.Dg,
                     a.Dg, a.qg + static_cast<size_t>(z) * a.nb * a.Dg, a.Dg, a.nb, a.Dg, a.D, m0, n0, 1.0f, false);
  } else {
    const int zk = z - nq;                   // index into [B, Hwk]
    const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
    const int b = zk / hwk, hk = zk % hwk;
    const int g = a.wk_per_kv ? hk : hk / a.group;
    gemm_tile<false>(a.kp + (static_cast<size_t>(b) * a.Hkv + g) * a.nb * 3 * a.D, 3 * a.D,
                     a.wk + static_cast<size_t>(hk) * 3 * a.D * a.Dg, a.Dg,
                     a.kg + static_cast<size_t>(zk) * a.nb * a.Dg, a.Dg, a.nb, a.Dg, 3 * a.D, m0, n0, 1.0f, false);
  }
}

__global__ __launch_bounds__(kGT) void gate_proj_kernel(GateArgs a) {
  // the K' projections (3D deep) are dispatched first, the Q' ones (D deep)
  // fill in after them
  const int nq = a.B * a.Hq, nk = static_cast<int>(gridDim.z) - nq;
  const int z = static_cast<int>(blockIdx.z) < nk ? nq + static_cast<int>(blockIdx.z) : static_cast<int>(blockIdx.z) - nk;
  gate_proj_body(a, blockIdx.x, blockIdx.y, z);
}

// Causal 64 x 64 tiles of the block logits z = Q' K'^T / sqrt(D). One
// workgroup per (row z = b * Hq + h, causal tile); ntri tiles per row.
// Workgroup w runs on XCD w % 8: when the rows split evenly over the 8 XCDs,
// XCD x takes whole rows z = x, x + 8, ... in turn, so each row's Q' and K'
// are fetched into one XCD's L2 instead of all eight.
__device__ __forceinline__ void gate_logits_body(const GateArgs& a, const int w, const int ntri) {
  const int nz = a.B * a.Hq;
  int z, idx;
  if (nz % 8 == 0) {
    const int i = w / 8;
    z = w % 8 + 8 * (i / ntri);
    idx = i % ntri;
  } else {
    z = w / ntri;
    idx = w % ntri;
  }
  // triangular decode of idx -> (ti, tj), tj <= ti
  int ti = static_cast<int>((sqrtf(8.0f * idx + 1.0f) - 1.0f) * 0.5f);
  while ((ti + 1) * (ti + 2) / 2 <= idx) ++ti;
  while (ti * (ti + 1) / 2 > idx) --ti;
  const int tj = idx - ti * (ti + 1) / 2;
  const int b = z / a.Hq, h = z % a.Hq;
  const int hk = a.wk_per_kv ? h / a.group : h;
  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  const float* Aq = a.qg + static_cast<size_t>(z) * a.nb * a.Dg;
  const float* Bk = a.kg + (static_cast<size_t>(b) * hwk + hk) * a.nb * a.Dg;
  float* C = a.scores + static_cast<size_t>(z) * a.nb * a.nb;
  gemm_tile<true>(Aq, a.Dg, Bk, a.Dg, C, a.nb, a.nb, a.nb, a.Dg, ti * kBM, tj * kBN, a.scale, true);
}

__global__ __launch_bounds__(kGT) void gate_logits_kernel(GateArgs a, int ntri) {
  gate_logits_body(a, blockIdx.x, ntri);
}

// ---------------------------------------------------------------------------
// Row softmax over j <= i, scores written back in place, then the mask.
// ---------------------------------------------------------------------------
constexpr int kST = 256;

__device__ __forceinline__ float block_reduce_max(float x, float* red) {
  x = wave_max(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kST / kWave; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float x, float* red) {
  x = wave_sum(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kST / kWave; ++w) r += red[w];
  return r;
}

// Softmax of the n logits in row[] (LDS; overwritten with the probabilities),
// written to srow[0 .. nb) (0 for j >= n) unless srow is null, then the mask
// mrow[0 .. nb): probability > threshold (mode 0) or the k largest (ties to the
// lower index, all n if k >= n); 0 for j >= n.
__device__ void softmax_mask_row(float* row, float* srow, uint8_t* mrow, int n, int nb, int mode, float threshold,
                                 int k) {
  __shared__ float red[kST / kWave];
  __shared__ int hist[256];
  __shared__ int sel_state[2];
  __shared__ int scan_tmp[kST / kWave];
  const int tid = threadIdx.x;

  float mx = -INFINITY;
  for (int j = tid; j < n; j += kST) mx = fmaxf(mx, row[j]);
  mx = block_reduce_max(mx, red);
  float sum = 0.f;
  for (int j = tid; j < n; j += kST) {
    const float e = expf(row[j] - mx);
    row[j] = e;
    sum += e;
  }
  sum = block_reduce_sum(sum, red);
  const float inv = 1.0f / sum;
  for (int j = tid; j < nb; j += kST) {
    float s = 0.f;
    if (j < n) {
      s = row[j] * inv;
      row[j] = s;
    }
    if (srow != nullptr) srow[j] = s;
  }
  __syncthreads();

  if (mode == 0) {
    for (int j = tid; j < nb; j += kST) mrow[j] = (j < n && row[j] > threshold) ? 1 : 0;
    return;
  }

  // ---- top-k --------------------------------------------------------------
  if (k >= n) {
    for (int j = tid; j < nb; j += kST) mrow[j] = j < n ? 1 : 0;
    return;
  }
  // radix select of the k-th largest value (probabilities are >= 0, so their
  // bit patterns order like the values)
  uint32_t prefix = 0, pmask = 0;
  int kk = k;
  const int lane = tid & 63, wave = tid >> 6;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;                           // kST == 256 bins
    __syncthreads();
    for (int j = tid; j < n; j += kST) {
      const uint32_t u = __float_as_uint(row[j]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane L owns bins 252-4L .. 255-4L (descending); suffix counts from the top
      int cnt4[4], own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { cnt4[e] = hist[255 - 4 * lane - e]; own += cnt4[e]; }
      const int inc = wave_inclusive_scan(own, lane);
      int above = inc - own;                 // count in bins higher than this lane's
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < kk && above + cnt4[e] >= kk) {
          sel_state[0] = 255 - 4 * lane - e;
          sel_state[1] = kk - above;
        }
        above += cnt4[e];
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(sel_state[0]) << shift;
    pmask |= 255u << shift;
    kk = sel_state[1];
    __syncthreads();
  }
  // keep every score above the k-th value, and the first kk equal to it by index
  const int chunk = (n + kST - 1) / kST;
  const int ja = tid * chunk, jb = min(n, ja + chunk);
  int eq = 0;
  for (int j = ja; j < jb; ++j) eq += (__float_as_uint(row[j]) == prefix);
  int inc = wave_inclusive_scan(eq, lane);
  if (lane == 63) scan_tmp[wave] = inc;
  __syncthreads();
  int before = inc - eq;
  for (int w = 0; w < wave; ++w) before += scan_tmp[w];
  for (int j = ja; j < jb; ++j) {
    const uint32_t u = __float_as_uint(row[j]);
    uint8_t keep = u > prefix ? 1 : 0;
    if (u == prefix) { keep = before < kk ? 1 : 0; ++before; }
    mrow[j] = keep;
  }
  for (int j = n + tid; j < nb; j += kST) mrow[j] = 0;
}

// Row i of head z: softmax over the causal logits j <= i (in place in the
// scores buffer) and the mask row.
__global__ __launch_bounds__(kST) void gate_softmax_mask_kernel(GateArgs a, TopkTable tk) {
  extern __shared__ float row[];             // nb floats
  const int i = blockIdx.x;
  const int z = blockIdx.y;                  // b * Hq + h
  const int n = i + 1;                       // causal entries of this row
  float* srow = a.scores + (static_cast<size_t>(z) * a.nb + i) * a.nb;
  for (int j = threadIdx.x; j < n; j += kST) row[j] = srow[j];
  __syncthreads();
  softmax_mask_row(row, a.skip_scores ? nullptr : srow, a.mask + (static_cast<size_t>(z) * a.nb + i) * a.nb, n,
                   a.nb, a.mode, a.threshold, tk.k[z % a.Hq]);
}

// This wave's LDS accesses so far have completed, and the compiler moves no
// memory access across the point.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int wave_max_int(int x) {
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Same row computation as gate_softmax_mask_kernel with one wavefront per row
// and the row in registers: lane l holds elements 256 t + 4 l + e (t < G,
// e < 4), so each load and store instruction covers 1 KiB of scores (256 B of
// mask) contiguous. Four independent rows per workgroup and no workgroup
// barrier: the reductions are cross-lane, the radix select's histogram is a
// per-wave LDS array. Rows up to 256 G blocks.
//
// Each element is carried as the bit pattern of its probability, with the
// entries past the causal end as -0.0 (sign bit set): no probability has that
// bit, so those entries never match a radix prefix (whose mask includes the
// sign bit) and compare below every probability as signed integers, and all
// the later steps are integer compares on the keys alone.
// The row's first n of nb entries are its logits (the rest are written as
// probability 0 and mask 0); k is its top-k count (mode 1); hist is this
// wavefront's 256-word LDS histogram. vec: the row's scores may be accessed
// as 16-byte groups and its mask bytes as 4-byte groups. store: write the
// probabilities back over the logits (else only the mask is written).
template <int G>
__device__ __forceinline__ void wave_softmax_mask_row(float* srow, uint8_t* mrow, int n, int nb, int mode,
                                                      float threshold, int k, bool vec, bool store, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  // 256-entry groups that hold causal entries (wave-uniform): the later ones
  // hold only -0.0 keys, which no count, histogram or maximum below can see,
  // so short rows skip them
  const int gn = (n + 255) >> 8;

  float v[G][4];                                        // logits; -inf past the causal end
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const int j0 = 256 * t + 4 * lane;
    if (vec && j0 + 3 < n) {
      const float4 x = *reinterpret_cast<const float4*>(srow + j0);
      v[t][0] = x.x; v[t][1] = x.y; v[t][2] = x.z; v[t][3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[t][e] = j0 + e < n ? srow[j0 + e] : -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < G; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, v[t][e]);
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < G; ++t) {
    if (t < gn) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = v[t][e] == -INFINITY ? -0.0f : expf(v[t][e] - mx);
        v[t][e] = x;
        sum += x;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[t][e] = -0.0f;
    }
  }
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
  uint32_t key[G][4];
#pragma unroll
  for (int t = 0; t < G; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) key[t][e] = __float_as_uint(v[t][e] * inv);
    if (!store) continue;
    const int j0 = 256 * t + 4 * lane;
    const float p0 = __uint_as_float(key[t][0] & 0x7fffffffu), p1 = __uint_as_float(key[t][1] & 0x7fffffffu);
    const float p2 = __uint_as_float(key[t][2] & 0x7fffffffu), p3 = __uint_as_float(key[t][3] & 0x7fffffffu);
    if (vec) {
      if (j0 < nb) *reinterpret_cast<float4*>(srow + j0) = make_float4(p0, p1, p2, p3);
    } else {
      if (j0 < nb) srow[j0] = p0;
      if (j0 + 1 < nb) srow[j0 + 1] = p1;
      if (j0 + 2 < nb) srow[j0 + 2] = p2;
      if (j0 + 3 < nb) srow[j0 + 3] = p3;
    }
  }

  // keep: key > lim as signed integers, plus (top-k) the first kk equal to lim
  int32_t lim = -1;                                     // every causal entry
  int kk = 0;
  if (mode == 0) {
    // p > T: bit patterns above T's for T > 0, above +0 for T = 0, every
    // entry for T < 0, none for a NaN T
    const float T = threshold;
    lim = T > 0.f ? static_cast<int32_t>(__float_as_uint(T)) : (T == 0.f ? 0 : (T < 0.f ? -1 : INT32_MAX));
  } else if (k < n) {
    // exact k-th largest probability (probabilities are >= 0: their bit
    // patterns order like the values). Its exponent field first, by binary
    // search on wave-wide counts of keys >= 2^e (ballots, no LDS); then the
    // mantissa 8 bits at a time from bit 22, with a per-wave LDS histogram in
    // which lane L owns bins 255-4L .. 252-4L.
    auto count_ge = [&](int32_t c) {
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < G; ++t)
        if (t < gn)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(static_cast<int32_t>(key[t][e]) >= c));
      return cnt;
    };
    int32_t kmax = INT32_MIN;
#pragma unroll
    for (int t = 0; t < G; ++t)
      if (t < gn)
#pragma unroll
        for (int e = 0; e < 4; ++e) kmax = max(kmax, static_cast<int32_t>(key[t][e]));
    int lo = 0, hi = wave_max_int(kmax) >> 23;          // count(>= 2^lo) = n >= k; the answer is <= hi
    // the k-th largest usually lies within 16 binades of the largest: one
    // count there first halves the search in that case (either branch keeps
    // the invariant, so the result is the same)
    if (hi > 16) {
      if (count_ge((hi - 16) << 23) >= k) lo = hi - 16;
      else hi = hi - 17;
    }
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (count_ge(mid << 23) >= k) lo = mid;
      else hi = mid - 1;
    }
    uint32_t prefix = static_cast<uint32_t>(lo) << 23, pmask = 0xff800000u;
    kk = k - count_ge((lo + 1) << 23);                  // how many of the exponent's bin to keep
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass < 2 ? 15 - 8 * pass : 0;
      const uint32_t width = pass < 2 ? 255u : 127u;
      *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0, 0, 0, 0);
      wave_lds_sync();
#pragma unroll
      for (int t = 0; t < G; ++t)
        if (t < gn)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((key[t][e] & pmask) == prefix) atomicAdd(&hist[(key[t][e] >> shift) & width], 1u);
      wave_lds_sync();
      const uint4 c4 = *reinterpret_cast<const uint4*>(hist + 252 - 4 * lane);
      const int cnt4[4] = {static_cast<int>(c4.w), static_cast<int>(c4.z), static_cast<int>(c4.y),
                           static_cast<int>(c4.x)};     // bins 255-4L, 254-4L, 253-4L, 252-4L
      const int own = cnt4[0] + cnt4[1] + cnt4[2] + cnt4[3];
      const int inc = wave_inclusive_scan(own, lane);
      int above = inc - own;                            // count in bins above this lane's
      int bin = 0, rem = 0;
      bool found = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < kk && above + cnt4[e] >= kk) {
          found = true;
          bin = 255 - 4 * lane - e;
          rem = kk - above;
        }
        above += cnt4[e];
      }
      const int src = static_cast<int>(__builtin_ctzll(__builtin_amdgcn_ballot_w64(found)));
      bin = __shfl(bin, src, kWave);
      kk = __shfl(rem, src, kWave);
      prefix |= static_cast<uint32_t>(bin) << shift;
      pmask |= width << shift;
      wave_lds_sync();                                  // the histogram is read before the next pass clears it
    }
    lim = static_cast<int32_t>(prefix);
    // when no more entries equal the k-th value than are kept, keep them all
    int eq_total = 0;
#pragma unroll
    for (int t = 0; t < G; ++t)
      if (t < gn)
#pragma unroll
        for (int e = 0; e < 4; ++e) eq_total += key[t][e] == prefix;
    if (wave_sum_int(eq_total) <= kk) {
      lim -= 1;                                         // > prefix - 1  <=>  >= prefix
      kk = 0;
    }
  }
  // the kk entries equal to lim with the lowest indices are kept as well
  int before = 0;                                       // such entries at lower indices
#pragma unroll
  for (int t = 0; t < G; ++t) {
    uint32_t keep = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) keep |= static_cast<uint32_t>(static_cast<int32_t>(key[t][e]) > lim) << (8 * e);
    if (kk > 0 && t < gn) {
      int eq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) eq += key[t][e] == static_cast<uint32_t>(lim);
      const int inc = wave_inclusive_scan(eq, lane);
      int b = before + inc - eq;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key[t][e] == static_cast<uint32_t>(lim)) {
          if (b < kk) keep |= 1u << (8 * e);
          ++b;
        }
      before += __shfl(inc, kWave - 1, kWave);
    }
    const int j0 = 256 * t + 4 * lane;
    if (vec) {
      if (j0 < nb) *reinterpret_cast<uint32_t*>(mrow + j0) = keep;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < nb) mrow[j0 + e] = static_cast<uint8_t>(keep >> (8 * e));
    }
  }
}

// Prefill rows: row i of head z has the causal entries j <= i.
template <int G>
__global__ __launch_bounds__(256) void gate_softmax_mask_wave_kernel(GateArgs a, TopkTable tk) {
  __shared__ __align__(16) uint32_t hist_all[4][256];
  // the row, its pointers and the access width are wave-uniform: scalar
  // addresses and branches
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const long long row = static_cast<long long>(blockIdx.x) * 4 + wave;
  if (row >= static_cast<long long>(a.B) * a.Hq * a.nb) return;
  const int z = static_cast<int>(row / a.nb), i = static_cast<int>(row - static_cast<long long>(z) * a.nb);
  // 16-byte score and 4-byte mask accesses when every row allows them (the
  // caller's maps need only 4-byte and 1-byte alignment)
  const bool vec = (a.nb & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0;
  wave_softmax_mask_row<G>(a.scores + static_cast<size_t>(row) * a.nb, a.mask + static_cast<size_t>(row) * a.nb,
                           i + 1, a.nb, a.mode, a.threshold, tk.k[z % a.Hq], vec, !a.skip_scores, hist_all[wave]);
}


// ---------------------------------------------------------------------------
// Decode-stage gate ("SeerAttention: Self-distilled Attention Gating for
// Efficient Long-context Prefilling", responses on decoding): no query
// pooling or projection; the compressed K cache holds the keys
// [max | min | avg]-pooled per block and projected by W_k (3D -> D).
// ---------------------------------------------------------------------------
// Compressed cache of blocks [block_begin, nb): one workgroup per (block,
// batch, W_k index, 32 output columns) pools the block's (up to 64) key rows
// of the KV head that W_k index reads, and projects the pool through its 32
// columns of W_k (3D -> D), the 3D-long sums split into 8 row ranges with
// eight independent accumulators each so many loads are in flight.
constexpr int kKcompCols = 32;
template <int D>
__global__ __launch_bounds__(256) void decode_kcomp_kernel(DecodeGateArgs a) {
  constexpr int NV = D / 8;                  // pooling: groups of 8 dims (16-byte loads)
  constexpr int P = 256 / NV;                // pooling: token parts
  constexpr int TPT = kBlock / P;            // pooling: tokens per thread
  constexpr int RP = 256 / kKcompCols;       // row ranges of the projection
  constexpr int RR = 3 * D / RP;             // rows per range
  __shared__ float red[3][P][D];
  __shared__ float kp[3 * D];
  __shared__ float part_s[RP][kKcompCols];
  const int j = a.block_begin + blockIdx.x;
  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  const int b = blockIdx.y / hwk, w = blockIdx.y - b * hwk;
  const int g = a.wk_per_kv ? w : w / a.group;
  const int n0 = blockIdx.z * kKcompCols;
  const int tid = threadIdx.x;
  {
    const int dg = tid % NV, part = tid / NV;
    const int t0 = j * kBlock, n_tok = min(kBlock, a.S - t0);
    const uint16_t* kr = a.k + ((static_cast<size_t>(b) * a.Hkv + g) * a.S + t0) * D + dg * 8;
    uint4 raw[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {            // all loads issued before use
      const int u = part + P * i;
      raw[i] = u < n_tok ? *reinterpret_cast<const uint4*>(kr + static_cast<size_t>(u) * D) : make_uint4(0, 0, 0, 0);
    }
    float mx[8], mn[8], sm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mx[e] = -INFINITY; mn[e] = INFINITY; sm[e] = 0.f; }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      if (part + P * i >= n_tok) continue;
      const uint32_t wv[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __uint_as_float((e & 1) ? (wv[e >> 1] & 0xffff0000u) : (wv[e >> 1] << 16));
        mx[e] = fmaxf(mx[e], x);
        mn[e] = fminf(mn[e], x);
        sm[e] += x;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[0][part][dg * 8 + e] = mx[e];
      red[1][part][dg * 8 + e] = mn[e];
      red[2][part][dg * 8 + e] = sm[e];
    }
    __syncthreads();
    if (tid < D) {
      float x0 = -INFINITY, x1 = INFINITY, x2 = 0.f;
      for (int p2 = 0; p2 < P; ++p2) {
        x0 = fmaxf(x0, red[0][p2][tid]);
        x1 = fminf(x1, red[1][p2][tid]);
        x2 += red[2][p2][tid];
      }
      kp[tid] = x0;
      kp[D + tid] = x1;
      kp[2 * D + tid] = x2 / static_cast<float>(n_tok);
    }
    __syncthreads();
  }
  const int col = tid % kKcompCols, rp = tid / kKcompCols;
  const float* wk = a.wk + static_cast<size_t>(w) * 3 * D * D + n0 + col;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int r0 = rp * RR;
#pragma unroll
  for (int r = 0; r < RR; r += 8)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(kp[r0 + r + e], wk[static_cast<size_t>(r0 + r + e) * D], acc[e]);
  part_s[rp][col] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (tid < kKcompCols) {
    float t = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < RP; ++p2) t += part_s[p2][tid];
    a.kcomp[((static_cast<size_t>(b) * hwk + w) * a.kcomp_blocks + j) * D + n0 + tid] = t;
  }
}

// Decode gate logits: 8 lanes per block (16-byte loads, 3 shuffle steps),
// 32 blocks per workgroup; workgroup (x, z) covers blocks 32x .. 32x+31 of
// query head z.
constexpr int kLogitBlocks = 32;
__global__ __launch_bounds__(256) void decode_logits_kernel(DecodeGateArgs a) {
  const int z = blockIdx.y;                  // b * Hq + h
  const int b = z / a.Hq, h = z - b * a.Hq;
  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  const int w = a.wk_per_kv ? h / a.group : h;
  const int sub = threadIdx.x & 7;           // lane within the block's 8
  const int j = blockIdx.x * kLogitBlocks + (threadIdx.x >> 3);
  const int dpl = a.D / 8;                   // dims per lane: 8 or 16
  float acc = 0.f;
  if (j < a.nb) {
    const float4* kr = reinterpret_cast<const float4*>(
        a.kcomp + ((static_cast<size_t>(b) * hwk + w) * a.kcomp_blocks + j) * a.D + sub * dpl);
    // the lane's dpl query values as 16-byte loads (8 bf16 each; q rows are
    // 16-byte aligned and dpl is 8 or 16)
    const uint4* qr = reinterpret_cast<const uint4*>(a.q + static_cast<size_t>(z) * a.D + sub * dpl);
    for (int i8 = 0; i8 < dpl / 8; ++i8) {
      const uint4 qv = qr[i8];
      const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 v = kr[2 * i8 + h];
        acc = fmaf(v.x, __uint_as_float(qw[2 * h] << 16), acc);
        acc = fmaf(v.y, __uint_as_float(qw[2 * h] & 0xffff0000u), acc);
        acc = fmaf(v.z, __uint_as_float(qw[2 * h + 1] << 16), acc);
        acc = fmaf(v.w, __uint_as_float(qw[2 * h + 1] & 0xffff0000u), acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (sub == 0 && j < a.nb) a.scores[static_cast<size_t>(z) * a.nb + j] = acc * a.scale;
}

// One workgroup per (batch, query head): softmax over every block, in place,
// and the mask.
// Decode rows: one workgroup of four wavefronts per row z = b * Hq + h (with
// one row per (batch, head) a single wavefront per row has too little work to
// hide its latency). The steps of wave_softmax_mask_row, with every maximum,
// count and histogram taken over the four wavefronts through LDS; wavefront w
// holds entries 1024 t + 256 w + 4 lane + e of the row, and every entry is
// valid (the newest token sees every cached block).
constexpr int kRowWaves = 4;
template <int G>
__global__ __launch_bounds__(kRowWaves * kWave) void decode_gate_kernel(DecodeGateArgs a, TopkTable tk) {
  __shared__ float redf[2][kRowWaves];
  __shared__ int redi[2][kRowWaves];
  __shared__ __align__(16) uint32_t hist[3][256];      // one per mantissa pass, zeroed up front
  __shared__ int tab[G][kRowWaves];                   // entries equal to the k-th value per 256-entry chunk
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int z = blockIdx.x;
  const int nb = a.nb;
  float* srow = a.scores + static_cast<size_t>(z) * nb;
  uint8_t* mrow = a.mask + static_cast<size_t>(z) * nb;
  // 16-byte score and 4-byte mask accesses when every row allows them
  const bool vec = (nb & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0;
  for (int i = threadIdx.x; i < 3 * 256; i += kRowWaves * kWave) hist[i >> 8][i & 255] = 0u;

  // workgroup-wide reductions, one barrier each: consecutive reductions use
  // alternate slots, so a slot is rewritten only after the next barrier
  int slot = 0;
  auto all_max = [&](float x) {
    x = wave_max(x);
    if (lane == 0) redf[slot][wave] = x;
    __syncthreads();
    const float r = fmaxf(fmaxf(redf[slot][0], redf[slot][1]), fmaxf(redf[slot][2], redf[slot][3]));
    slot ^= 1;
    return r;
  };
  auto all_sum = [&](float x) {
    x = wave_sum(x);
    if (lane == 0) redf[slot][wave] = x;
    __syncthreads();
    const float r = (redf[slot][0] + redf[slot][1]) + (redf[slot][2] + redf[slot][3]);
    slot ^= 1;
    return r;
  };
  auto all_max_int = [&](int x) {                     // x: wave-uniform or per lane
    x = wave_max_int(x);
    if (lane == 0) redi[slot][wave] = x;
    __syncthreads();
    const int r = max(max(redi[slot][0], redi[slot][1]), max(redi[slot][2], redi[slot][3]));
    slot ^= 1;
    return r;
  };
  auto all_add_int = [&](int x) {                     // x: wave-uniform
    if (lane == 0) redi[slot][wave] = x;
    __syncthreads();
    const int r = redi[slot][0] + redi[slot][1] + redi[slot][2] + redi[slot][3];
    slot ^= 1;
    return r;
  };

  float v[G][4];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const int j0 = 1024 * t + 256 * wave + 4 * lane;
    if (vec && j0 + 3 < nb) {
      const float4 x = *reinterpret_cast<const float4*>(srow + j0);
      v[t][0] = x.x; v[t][1] = x.y; v[t][2] = x.z; v[t][3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[t][e] = j0 + e < nb ? srow[j0 + e] : -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < G; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, v[t][e]);
  mx = all_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < G; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = v[t][e] == -INFINITY ? -0.0f : expf(v[t][e] - mx);
      v[t][e] = x;
      sum += x;
    }
  sum = all_sum(sum);
  const float inv = 1.0f / sum;
  uint32_t key[G][4];                                 // probability bit patterns; -0 past the row
#pragma unroll
  for (int t = 0; t < G; ++t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) key[t][e] = __float_as_uint(v[t][e] * inv);
    const int j0 = 1024 * t + 256 * wave + 4 * lane;
    const float p0 = __uint_as_float(key[t][0] & 0x7fffffffu), p1 = __uint_as_float(key[t][1] & 0x7fffffffu);
    const float p2 = __uint_as_float(key[t][2] & 0x7fffffffu), p3 = __uint_as_float(key[t][3] & 0x7fffffffu);
    if (vec) {
      if (j0 < nb) *reinterpret_cast<float4*>(srow + j0) = make_float4(p0, p1, p2, p3);
    } else {
      if (j0 < nb) srow[j0] = p0;
      if (j0 + 1 < nb) srow[j0 + 1] = p1;
      if (j0 + 2 < nb) srow[j0 + 2] = p2;
      if (j0 + 3 < nb) srow[j0 + 3] = p3;
    }
  }

  // keep: key > lim as signed integers, plus (top-k) the first kk equal to lim
  const int k = tk.k[z % a.Hq];
  int32_t lim = -1;                                   // every entry
  int kk = 0;
  if (a.mode == 0) {
    const float T = a.threshold;
    lim = T > 0.f ? static_cast<int32_t>(__float_as_uint(T)) : (T == 0.f ? 0 : (T < 0.f ? -1 : INT32_MAX));
  } else if (k < nb) {
    // exponent of the k-th largest probability by binary search on counts of
    // keys >= 2^e, then its mantissa 8 bits at a time from bit 22
    auto count_ge = [&](int32_t c) {
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(static_cast<int32_t>(key[t][e]) >= c));
      return all_add_int(cnt);
    };
    int32_t kmax = INT32_MIN;
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) kmax = max(kmax, static_cast<int32_t>(key[t][e]));
    int lo = 0, hi = all_max_int(kmax) >> 23;           // count(>= 2^lo) = nb >= k; the answer is <= hi
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (count_ge(mid << 23) >= k) lo = mid;
      else hi = mid - 1;
    }
    uint32_t prefix = static_cast<uint32_t>(lo) << 23, pmask = 0xff800000u;
    kk = k - count_ge((lo + 1) << 23);
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass < 2 ? 15 - 8 * pass : 0;
      const uint32_t width = pass < 2 ? 255u : 127u;
      uint32_t* h = hist[pass];
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((key[t][e] & pmask) == prefix) atomicAdd(&h[(key[t][e] >> shift) & width], 1u);
      __syncthreads();
      // every wavefront reads the whole histogram and takes the same bin;
      // lane L owns bins 255-4L .. 252-4L
      const uint4 c4 = *reinterpret_cast<const uint4*>(h + 252 - 4 * lane);
      const int cnt4[4] = {static_cast<int>(c4.w), static_cast<int>(c4.z), static_cast<int>(c4.y),
                           static_cast<int>(c4.x)};
      const int own = cnt4[0] + cnt4[1] + cnt4[2] + cnt4[3];
      const int inc = wave_inclusive_scan(own, lane);
      int above = inc - own;
      int bin = 0, rem = 0;
      bool found = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < kk && above + cnt4[e] >= kk) {
          found = true;
          bin = 255 - 4 * lane - e;
          rem = kk - above;
        }
        above += cnt4[e];
      }
      const int src = static_cast<int>(__builtin_ctzll(__builtin_amdgcn_ballot_w64(found)));
      bin = __shfl(bin, src, kWave);
      kk = __shfl(rem, src, kWave);
      prefix |= static_cast<uint32_t>(bin) << shift;
      pmask |= width << shift;
    }
    lim = static_cast<int32_t>(prefix);
    int eq = 0;
#pragma unroll
    for (int t = 0; t < G; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) eq += key[t][e] == prefix;
    if (all_add_int(wave_sum_int(eq)) <= kk) {        // no more equal to the k-th value than are kept
      lim -= 1;
      kk = 0;
    }
  }
  // the kk entries equal to lim with the lowest indices are kept as well:
  // count them per 256-entry chunk first
  if (kk > 0) {
#pragma unroll
    for (int t = 0; t < G; ++t) {
      int eq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) eq += key[t][e] == static_cast<uint32_t>(lim);
      eq = wave_sum_int(eq);
      if (lane == 0) tab[t][wave] = eq;
    }
    __syncthreads();
  }
  int before = 0;                                     // equal entries in the chunks before this one
#pragma unroll
  for (int t = 0; t < G; ++t) {
    uint32_t keep = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) keep |= static_cast<uint32_t>(static_cast<int32_t>(key[t][e]) > lim) << (8 * e);
    if (kk > 0) {
      int b0 = before;
      for (int w = 0; w < wave; ++w) b0 += tab[t][w];
      int eq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) eq += key[t][e] == static_cast<uint32_t>(lim);
      const int inc = wave_inclusive_scan(eq, lane);
      int b = b0 + inc - eq;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key[t][e] == static_cast<uint32_t>(lim)) {
          if (b < kk) keep |= 1u << (8 * e);
          ++b;
        }
      before += tab[t][0] + tab[t][1] + tab[t][2] + tab[t][3];
    }
    const int j0 = 1024 * t + 256 * wave + 4 * lane;
    if (vec) {
      if (j0 < nb) *reinterpret_cast<uint32_t*>(mrow + j0) = keep;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < nb) mrow[j0 + e] = static_cast<uint8_t>(keep >> (8 * e));
    }
  }
}

// ---------------------------------------------------------------------------
// Block-level RoPE ("SeerAttention: Learning Intrinsic Sparse Attention in
// Your LLMs", explainer section 3.4, "Block-Level RoPE"): the projected Q' and
// K' rows are rotated at their block position i with base theta' = theta / 64,
// dims d and d + Dg/2 forming a pair: angle = i * theta'^(-2d/Dg). In place,
// one thread per (row, pair); the angle, its sine and cosine and the rotation
// are computed in fp64 so that long sequences keep the angle exact. `sign` =
// -1 rotates back (the transpose, used by the gradient).
// ---------------------------------------------------------------------------
constexpr int kRopeRows = 8;               // rows rotated per thread with one angle
// rows kRopeRows zy .. of x [rows][nb][dg]: one thread per (block position i,
// pair d) computes the fp64 angle once and rotates that pair in each row
__device__ __forceinline__ void rope_rows(float* __restrict__ x, int rows, int nb, int dg, double base, double sign,
                                          int zy) {
  const int half = dg / 2;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;   // over nb * half
  if (idx >= static_cast<long long>(nb) * half) return;
  const int i = static_cast<int>(idx / half), d = static_cast<int>(idx - static_cast<long long>(i) * half);
  const double ang = sign * static_cast<double>(i) * pow(base, -2.0 * d / dg);
  double sn, cs;
  sincos(ang, &sn, &cs);
  const int z0 = zy * kRopeRows;
  float x1[kRopeRows], x2[kRopeRows];
#pragma unroll
  for (int u = 0; u < kRopeRows; ++u) {
    const float* r = x + (static_cast<size_t>(min(z0 + u, rows - 1)) * nb + i) * dg;
    x1[u] = r[d];
    x2[u] = r[d + half];
  }
#pragma unroll
  for (int u = 0; u < kRopeRows; ++u) {
    if (z0 + u >= rows) break;
    float* r = x + (static_cast<size_t>(z0 + u) * nb + i) * dg;
    r[d] = static_cast<float>(static_cast<double>(x1[u]) * cs - static_cast<double>(x2[u]) * sn);
    r[d + half] = static_cast<float>(static_cast<double>(x2[u]) * cs + static_cast<double>(x1[u]) * sn);
  }
}

// Q' (rows0 rows at x0) and K' (rows1 rows at x1) in one launch: grid.y
// covers x0's row groups, then x1's
__global__ __launch_bounds__(256) void gate_rope_kernel(float* __restrict__ x0, int rows0, float* __restrict__ x1,
                                                        int rows1, int nb, int dg, double base, double sign) {
  const int ty0 = (rows0 + kRopeRows - 1) / kRopeRows;
  const int zy = static_cast<int>(blockIdx.y);
  if (zy < ty0) rope_rows(x0, rows0, nb, dg, base, sign, zy);
  else rope_rows(x1, rows1, nb, dg, base, sign, zy - ty0);
}

// ---------------------------------------------------------------------------
// Self-distillation step (same page, "Training Procedure": loss =
// D_KL(gt || score)). One workgroup per row (b, h, i) of the block logits z:
// with p = gt row / its sum and log score = z - logsumexp(z) over j <= i,
//   row_loss = sum_{p_j > 0} p_j (log p_j - log score_j),
//   dz_j = (score_j - p_j) / (B Hq nb) for j <= i, 0 above the diagonal,
// dz overwriting the logits in place. A row whose ground truth sums to 0 has
// no target distribution and contributes nothing (loss 0, dz 0).
// ---------------------------------------------------------------------------
// gate_kl_kernel with one wavefront per row (rows up to 256 G blocks), the
// row in registers in the layout of gate_softmax_mask_wave_kernel. Entries
// past the causal end load as logit -inf and gt 0, so they drop out of every
// sum and their dz is 0 without a per-element test.
template <int G>
__global__ __launch_bounds__(256) void gate_kl_wave_kernel(GateArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));   // wave-uniform row
  const int lane = threadIdx.x & 63;
  const long long row = static_cast<long long>(blockIdx.x) * 4 + wave;
  if (row >= static_cast<long long>(a.B) * a.Hq * a.nb) return;
  const int nb = a.nb;
  const int i = static_cast<int>(row % nb);
  const int n = i + 1;
  float* zrow = a.scores + static_cast<size_t>(row) * nb;
  const float* grow = a.gt + static_cast<size_t>(row) * nb;
  // 16-byte accesses when every row allows them (gt needs only 4-byte
  // alignment)
  const bool vec = (nb & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.scores) | reinterpret_cast<uintptr_t>(a.gt)) & 15) == 0;
  float zv[G][4], gv[G][4];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    const int j0 = 256 * t + 4 * lane;
    if (vec && j0 + 3 < n) {
      const float4 x = *reinterpret_cast<const float4*>(zrow + j0);
      const float4 y = *reinterpret_cast<const float4*>(grow + j0);
      zv[t][0] = x.x; zv[t][1] = x.y; zv[t][2] = x.z; zv[t][3] = x.w;
      gv[t][0] = y.x; gv[t][1] = y.y; gv[t][2] = y.z; gv[t][3] = y.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        zv[t][e] = j0 + e < n ? zrow[j0 + e] : -INFINITY;
        gv[t][e] = j0 + e < n ? grow[j0 + e] : 0.f;
      }
    }
  }
  float mx = -INFINITY, gsum = 0.f;
#pragma unroll
  for (int t = 0; t < G; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx = fmaxf(mx, zv[t][e]);
      gsum += gv[t][e];
    }
  mx = wave_max(mx);
  gsum = wave_sum(gsum);
  // 256-entry groups holding causal entries (wave-uniform); the later ones
  // add nothing to l or the loss and take dz = 0
  const int gn = (n + 255) >> 8;
  float l = 0.f;
#pragma unroll
  for (int t = 0; t < G; ++t)
    if (t < gn)
#pragma unroll
      for (int e = 0; e < 4; ++e) l += expf(zv[t][e] - mx);
  l = wave_sum(l);
  const float lse = mx + logf(l);
  const bool valid = gsum > 0.f;             // a row without ground-truth mass contributes nothing
  const float inv_g = valid ? 1.0f / gsum : 0.f;
  const float inv_rows = 1.0f / (static_cast<float>(a.B) * a.Hq * a.nb);
  float kl = 0.f;
#pragma unroll
  for (int t = 0; t < G; ++t) {
    float dz[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < gn) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ls = zv[t][e] - lse;
        const float pj = gv[t][e] * inv_g;
        if (pj > 0.f) kl += pj * (logf(pj) - ls);
        dz[e] = valid ? (expf(ls) - pj) * inv_rows : 0.f;
      }
    }
    const int j0 = 256 * t + 4 * lane;
    if (vec) {
      if (j0 < nb) *reinterpret_cast<float4*>(zrow + j0) = make_float4(dz[0], dz[1], dz[2], dz[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < nb) zrow[j0 + e] = dz[e];
    }
  }
  kl = wave_sum(kl);
  if (lane == 0) a.row_loss[row] = kl;
}

__global__ __launch_bounds__(kST) void gate_kl_kernel(GateArgs a) {
  __shared__ float red[kST / kWave];
  const int i = blockIdx.x;
  const int z = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = i + 1;
  float* zrow = a.scores + (static_cast<size_t>(z) * a.nb + i) * a.nb;
  const float* grow = a.gt + (static_cast<size_t>(z) * a.nb + i) * a.nb;
  float mx = -INFINITY, gsum = 0.f;
  for (int j = tid; j < n; j += kST) {
    mx = fmaxf(mx, zrow[j]);
    gsum += grow[j];
  }
  mx = block_reduce_max(mx, red);
  gsum = block_reduce_sum(gsum, red);
  float l = 0.f;
  for (int j = tid; j < n; j += kST) l += expf(zrow[j] - mx);
  l = block_reduce_sum(l, red);
  const float lse = mx + logf(l);
  const bool valid = gsum > 0.f;             // a row without ground-truth mass contributes nothing
  const float inv_g = valid ? 1.0f / gsum : 0.f;
  const float inv_rows = 1.0f / (static_cast<float>(a.B) * a.Hq * a.nb);
  float kl = 0.f;
  for (int j = tid; j < a.nb; j += kST) {
    float dz = 0.f;
    if (j < n) {
      const float ls = zrow[j] - lse;
      const float pj = grow[j] * inv_g;
      if (pj > 0.f) kl += pj * (logf(pj) - ls);
      dz = valid ? (expf(ls) - pj) * inv_rows : 0.f;
    }
    zrow[j] = dz;
  }
  kl = block_reduce_sum(kl, red);
  if (tid == 0) a.row_loss[static_cast<size_t>(z) * a.nb + i] = kl;
}

// dQ'[z] = dz[z] K'[b, hk] / sqrt(D) and dK'[z] = dz[z]^T Q'[z] / sqrt(D) for
// every query head z = b Hq + h (dz lower triangular: the k range is cut to
// the causal part). blockIdx.z < B Hq: dQ', else dK'.
__global__ __launch_bounds__(kGT) void gate_dproj_kernel(GateArgs a) {
  const int nq = a.B * a.Hq;
  const int zz = blockIdx.z;
  const int z = zz < nq ? zz : zz - nq;
  const int b = z / a.Hq, h = z % a.Hq;
  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  const int hk = a.wk_per_kv ? h / a.group : h;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
  const float* dz = a.scores + static_cast<size_t>(z) * a.nb * a.nb;
  f32x16_t acc = {};
  if (zz < nq) {
    const float* kg = a.kg + (static_cast<size_t>(b) * hwk + hk) * a.nb * a.Dg;
    gemm_accum<false, false>(acc, dz, a.nb, kg, a.Dg, a.nb, a.Dg, 0, min(a.nb, m0 + kBM), m0, n0);
    gemm_store(acc, a.dqg + static_cast<size_t>(z) * a.nb * a.Dg, a.Dg, a.nb, a.Dg, m0, n0, a.scale, false);
  } else {
    const float* qg = a.qg + static_cast<size_t>(z) * a.nb * a.Dg;
    gemm_accum<true, false>(acc, dz, a.nb, qg, a.Dg, a.nb, a.Dg, m0 / kBK * kBK, a.nb, m0, n0);
    gemm_store(acc, a.dkg + static_cast<size_t>(z) * a.nb * a.Dg, a.Dg, a.nb, a.Dg, m0, n0, a.scale, false);
  }
}

// Weight gradients: dW_q[h] = sum_b Qp[b,h]^T dQ'[b,h] (D x Dg) and
// dW_k[w] = sum_b sum_{h -> w} Kp[b,g(h)]^T dK'[b,h] (3D x Dg), where h -> w
// are the query heads using W_k[w] (one, or the G heads of KV group w).
// blockIdx.z < Hq: W_q of head z, else W_k index z - Hq.
__global__ __launch_bounds__(kGT) void gate_dweight_kernel(GateArgs a) {
  const int zz = blockIdx.z;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
  f32x16_t acc = {};
  if (zz < a.Hq) {
    if (m0 >= a.D) return;                   // uniform per workgroup
    for (int b = 0; b < a.B; ++b) {
      const size_t zq = static_cast<size_t>(b) * a.Hq + zz;
      gemm_accum<true, false>(acc, a.qp + zq * a.nb * a.D, a.D, a.dqg + zq * a.nb * a.Dg, a.Dg, a.D, a.Dg, 0,
                              a.nb, m0, n0);
    }
    gemm_store(acc, a.grad_wq + static_cast<size_t>(zz) * a.D * a.Dg, a.Dg, a.D, a.Dg, m0, n0, 1.0f, false);
  } else {
    const int w = zz - a.Hq;
    const int K3 = 3 * a.D;
    if (m0 >= K3) return;
    const int h0 = a.wk_per_kv ? w * a.group : w, h1 = a.wk_per_kv ? h0 + a.group : w + 1;
    for (int b = 0; b < a.B; ++b)
      for (int h = h0; h < h1; ++h) {
        const int g = h / a.group;
        const size_t zq = static_cast<size_t>(b) * a.Hq + h;
        gemm_accum<true, false>(acc, a.kp + (static_cast<size_t>(b) * a.Hkv + g) * a.nb * K3, K3,
                                a.dkg + zq * a.nb * a.Dg, a.Dg, K3, a.Dg, 0, a.nb, m0, n0);
      }
    gemm_store(acc, a.grad_wk + static_cast<size_t>(w) * K3 * a.Dg, a.Dg, K3, a.Dg, m0, n0, 1.0f, false);
  }
}

// loss = mean of the row divergences, in fp64 and a fixed order (bitwise
// repeatable), by one workgroup: thread t
// adds rows t, t + 1024, ... in turn with 16 loads in flight, then a fixed
// tree over the threads.
constexpr int kLossThreads = 1024;
__global__ __launch_bounds__(kLossThreads) void gate_loss_kernel(GateArgs a) {
  __shared__ double red[kLossThreads];
  const long long n = static_cast<long long>(a.B) * a.Hq * a.nb;
  double s = 0.0;
  for (long long r0 = threadIdx.x; r0 < n; r0 += 16 * kLossThreads) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = r0 + u * kLossThreads < n ? a.row_loss[r0 + u * kLossThreads] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (r0 + u * kLossThreads < n) s += v[u];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kLossThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.loss[0] = static_cast<float>(red[0] / static_cast<double>(n));
}

// ---------------------------------------------------------------------------
// A packed batch's gate, one launch per stage (GateVarlenTable). Every
// workgroup (softmax: every wavefront) finds its sequence by binary search in
// a prefix table and runs the batch-1 code on that sequence's view, so each
// sequence's scores and mask are bitwise those of its own batch-1 call.
// ---------------------------------------------------------------------------
// last s in [0, n) with p[s] <= x
__device__ __forceinline__ int varlen_seq(const int* p, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// the batch-1 arguments of sequence s of the run
__device__ __forceinline__ GateArgs gate_seq(const GateArgs& a, const GateVarlenTable& t, int s) {
  GateArgs r = a;
  const size_t t0 = static_cast<size_t>(t.tokp[s]);
  const size_t b0 = static_cast<size_t>(t.nbp[s]);
  const size_t hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  r.q = a.q + t0 * a.D;
  r.k = a.k + t0 * a.D;
  r.S = t.tokp[s + 1] - t.tokp[s];
  r.nb = t.nbp[s + 1] - t.nbp[s];
  r.qp = a.qp + b0 * a.Hq * a.D;
  r.kp = a.kp + b0 * a.Hkv * 3 * a.D;
  r.qg = a.qg + b0 * a.Hq * a.Dg;
  r.kg = a.kg + b0 * hwk * a.Dg;
  r.scores = a.scores + t.mp[s] * a.Hq;
  r.mask = a.mask + t.mp[s] * a.Hq;
  return r;
}

template <int D>
__global__ __launch_bounds__(kPoolThreads) void gate_pool_varlen_kernel(GateArgs a, GateVarlenTable t) {
  const int s = varlen_seq(t.nbp, t.n, blockIdx.x);
  gate_pool_body<D>(gate_seq(a, t, s), blockIdx.x - t.nbp[s], blockIdx.y);
}

__global__ __launch_bounds__(kGT) void gate_proj_varlen_kernel(GateArgs a, GateVarlenTable t) {
  const int s = varlen_seq(t.pp, t.n, blockIdx.x);
  gate_proj_body(gate_seq(a, t, s), blockIdx.x - t.pp[s], blockIdx.y, blockIdx.z);
}

// as gate_rope_kernel over the run: x holds each sequence's [rows, nb, dg]
// part one after another; the thread index runs over all blocks' pairs
__global__ __launch_bounds__(256) void gate_rope_varlen_kernel(float* __restrict__ x, int rows, GateVarlenTable t,
                                                               int dg, double base, double sign) {
  const int half = dg / 2;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long long>(t.nbp[t.n]) * half) return;
  const int gi = static_cast<int>(idx / half), d = static_cast<int>(idx - static_cast<long long>(gi) * half);
  const int s = varlen_seq(t.nbp, t.n, gi);
  const int i = gi - t.nbp[s], nb = t.nbp[s + 1] - t.nbp[s];
  float* xs = x + static_cast<size_t>(t.nbp[s]) * rows * dg;
  const double ang = sign * static_cast<double>(i) * pow(base, -2.0 * d / dg);
  double sn, cs;
  sincos(ang, &sn, &cs);
  const int z0 = blockIdx.y * kRopeRows;
  float x1[kRopeRows], x2[kRopeRows];
#pragma unroll
  for (int u = 0; u < kRopeRows; ++u) {
    const float* r = xs + (static_cast<size_t>(min(z0 + u, rows - 1)) * nb + i) * dg;
    x1[u] = r[d];
    x2[u] = r[d + half];
  }
#pragma unroll
  for (int u = 0; u < kRopeRows; ++u) {
    if (z0 + u >= rows) break;
    float* r = xs + (static_cast<size_t>(z0 + u) * nb + i) * dg;
    r[d] = static_cast<float>(static_cast<double>(x1[u]) * cs - static_cast<double>(x2[u]) * sn);
    r[d + half] = static_cast<float>(static_cast<double>(x2[u]) * cs + static_cast<double>(x1[u]) * sn);
  }
}

__global__ __launch_bounds__(kGT) void gate_logits_varlen_kernel(GateArgs a, GateVarlenTable t) {
  const int s = varlen_seq(t.lp, t.n, blockIdx.x);
  const int T = (t.nbp[s + 1] - t.nbp[s] + kBM - 1) / kBM;
  gate_logits_body(gate_seq(a, t, s), blockIdx.x - t.lp[s], T * (T + 1) / 2);
}

// rows of the run: sequence s holds rows Hq nbp[s] .. Hq nbp[s+1], head major
template <int G>
__global__ __launch_bounds__(256) void gate_softmax_mask_varlen_kernel(GateArgs a, TopkTable tk, GateVarlenTable t) {
  __shared__ __align__(16) uint32_t hist_all[4][256];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int row = static_cast<int>(blockIdx.x) * 4 + wave;
  if (row >= a.Hq * t.nbp[t.n]) return;
  const int s = varlen_seq(t.nbp, t.n, row / a.Hq);
  const GateArgs b = gate_seq(a, t, s);
  const int local = row - a.Hq * t.nbp[s];
  const int z = local / b.nb, i = local - z * b.nb;
  const bool vec = (b.nb & 3) == 0 && (reinterpret_cast<uintptr_t>(b.scores) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(b.mask) & 3) == 0;
  wave_softmax_mask_row<G>(b.scores + static_cast<size_t>(local) * b.nb, b.mask + static_cast<size_t>(local) * b.nb,
                           i + 1, b.nb, b.mode, b.threshold, tk.k[z], vec, !b.skip_scores, hist_all[wave]);
}

hipError_t launch_rope(const GateArgs& a, float* x0, int rows0, float* x1, int rows1, double sign, hipStream_t st) {
  const long long n = static_cast<long long>(a.nb) * (a.Dg / 2);
  dim3 g(static_cast<unsigned>((n + 255) / 256), (rows0 + kRopeRows - 1) / kRopeRows + (rows1 + kRopeRows - 1) / kRopeRows);
  hipLaunchKernelGGL(gate_rope_kernel, g, dim3(256), 0, st, x0, rows0, x1, rows1, a.nb, a.Dg, a.rope_base, sign);
  return hipGetLastError();
}

// pool, projections, optional block RoPE, causal logits (shared by both calls)
hipError_t launch_gate_logits(const GateArgs& a, hipStream_t st) {
  const int H = a.Hq + a.Hkv;
  dim3 gp(a.nb, a.B * H);
  if (a.D == 64) hipLaunchKernelGGL(gate_pool_kernel<64>, gp, dim3(kPoolThreads), 0, st, a);
  else hipLaunchKernelGGL(gate_pool_kernel<128>, gp, dim3(kPoolThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  dim3 gj((a.nb + kBM - 1) / kBM, (a.Dg + kBN - 1) / kBN, a.B * a.Hq + a.B * hwk);
  hipLaunchKernelGGL(gate_proj_kernel, gj, dim3(kGT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  if (a.rope_base > 0.0) {
    if ((e = launch_rope(a, a.qg, a.B * a.Hq, a.kg, a.B * hwk, 1.0, st)) != hipSuccess) return e;
  }

  const int T = (a.nb + kBM - 1) / kBM;
  const int ntri = T * (T + 1) / 2;
  const long long nwg = static_cast<long long>(ntri) * a.B * a.Hq;
  // a 1D grid holds fewer than 2^32 work-items (any score map that fits in
  // device memory is far below this)
  if (nwg * kGT > 0xffffffffLL) return hipErrorInvalidValue;
  const dim3 gl(static_cast<unsigned>(nwg));
  hipLaunchKernelGGL(gate_logits_kernel, gl, dim3(kGT), 0, st, a, ntri);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate(const GateArgs& a, const TopkTable& tk, hipStream_t st) {
  hipError_t e = launch_gate_logits(a, st);
  if (e != hipSuccess) return e;
  const long long rows = static_cast<long long>(a.B) * a.Hq * a.nb;
  const dim3 gw(static_cast<unsigned>((rows + 3) / 4));
  if (a.nb <= 256) hipLaunchKernelGGL(gate_softmax_mask_wave_kernel<1>, gw, dim3(256), 0, st, a, tk);
  else if (a.nb <= 512) hipLaunchKernelGGL(gate_softmax_mask_wave_kernel<2>, gw, dim3(256), 0, st, a, tk);
  else if (a.nb <= 1024) hipLaunchKernelGGL(gate_softmax_mask_wave_kernel<4>, gw, dim3(256), 0, st, a, tk);
  else if (a.nb <= 2048) hipLaunchKernelGGL(gate_softmax_mask_wave_kernel<8>, gw, dim3(256), 0, st, a, tk);
  else if (a.nb <= 4096) hipLaunchKernelGGL(gate_softmax_mask_wave_kernel<16>, gw, dim3(256), 0, st, a, tk);
  else {
    dim3 gs(a.nb, a.B * a.Hq);
    hipLaunchKernelGGL(gate_softmax_mask_kernel, gs, dim3(kST), static_cast<size_t>(a.nb) * sizeof(float), st, a, tk);
  }
  return hipGetLastError();
}

hipError_t launch_gate_varlen(const GateArgs& a, const TopkTable& tk, const GateVarlenTable& t, int max_nb,
                              hipStream_t st) {
  if (t.n < 1 || t.n > kGateVarlenMaxSeqs || max_nb > kGateVarlenMaxBlocks || a.B != 1) return hipErrorInvalidValue;
  const int nbt = t.nbp[t.n];
  const dim3 gp(nbt, a.Hq + a.Hkv);
  if (a.D == 64) hipLaunchKernelGGL(gate_pool_varlen_kernel<64>, gp, dim3(kPoolThreads), 0, st, a, t);
  else hipLaunchKernelGGL(gate_pool_varlen_kernel<128>, gp, dim3(kPoolThreads), 0, st, a, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  hipLaunchKernelGGL(gate_proj_varlen_kernel, dim3(t.pp[t.n], (a.Dg + kBN - 1) / kBN, a.Hq + hwk), dim3(kGT), 0, st,
                     a, t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.rope_base > 0.0) {
    const long long n = static_cast<long long>(nbt) * (a.Dg / 2);
    const unsigned gx = static_cast<unsigned>((n + 255) / 256);
    hipLaunchKernelGGL(gate_rope_varlen_kernel, dim3(gx, (a.Hq + kRopeRows - 1) / kRopeRows), dim3(256), 0, st, a.qg,
                       a.Hq, t, a.Dg, a.rope_base, 1.0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gate_rope_varlen_kernel, dim3(gx, (hwk + kRopeRows - 1) / kRopeRows), dim3(256), 0, st, a.kg,
                       hwk, t, a.Dg, a.rope_base, 1.0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gate_logits_varlen_kernel, dim3(t.lp[t.n]), dim3(kGT), 0, st, a, t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long rows = static_cast<long long>(a.Hq) * nbt;
  const dim3 gw(static_cast<unsigned>((rows + 3) / 4));
  if (max_nb <= 256) hipLaunchKernelGGL(gate_softmax_mask_varlen_kernel<1>, gw, dim3(256), 0, st, a, tk, t);
  else if (max_nb <= 512) hipLaunchKernelGGL(gate_softmax_mask_varlen_kernel<2>, gw, dim3(256), 0, st, a, tk, t);
  else if (max_nb <= 1024) hipLaunchKernelGGL(gate_softmax_mask_varlen_kernel<4>, gw, dim3(256), 0, st, a, tk, t);
  else if (max_nb <= 2048) hipLaunchKernelGGL(gate_softmax_mask_varlen_kernel<8>, gw, dim3(256), 0, st, a, tk, t);
  else hipLaunchKernelGGL(gate_softmax_mask_varlen_kernel<16>, gw, dim3(256), 0, st, a, tk, t);
  return hipGetLastError();
}

hipError_t launch_decode_kcomp(const DecodeGateArgs& a, hipStream_t st) {
  dim3 g(a.nb - a.block_begin, a.B * (a.wk_per_kv ? a.Hkv : a.Hq), a.D / kKcompCols);
  if (a.D == 64) hipLaunchKernelGGL(decode_kcomp_kernel<64>, g, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(decode_kcomp_kernel<128>, g, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_gate(const DecodeGateArgs& a, const TopkTable& tk, hipStream_t st) {
  hipLaunchKernelGGL(decode_logits_kernel, dim3((a.nb + kLogitBlocks - 1) / kLogitBlocks, a.B * a.Hq), dim3(256), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.B * a.Hq), block(kRowWaves * kWave);
  if (a.nb <= 1024) hipLaunchKernelGGL(decode_gate_kernel<1>, grid, block, 0, st, a, tk);
  else if (a.nb <= 2048) hipLaunchKernelGGL(decode_gate_kernel<2>, grid, block, 0, st, a, tk);
  else if (a.nb <= 4096) hipLaunchKernelGGL(decode_gate_kernel<4>, grid, block, 0, st, a, tk);
  else if (a.nb <= 8192) hipLaunchKernelGGL(decode_gate_kernel<8>, grid, block, 0, st, a, tk);
  else hipLaunchKernelGGL(decode_gate_kernel<16>, grid, block, 0, st, a, tk);
  return hipGetLastError();
}

hipError_t launch_gate_distill(const GateArgs& a, hipStream_t st) {
  hipError_t e = launch_gate_logits(a, st);
  if (e != hipSuccess) return e;
  {
    const long long rows = static_cast<long long>(a.B) * a.Hq * a.nb;
    const dim3 gw(static_cast<unsigned>((rows + 3) / 4));
    if (a.nb <= 256) hipLaunchKernelGGL(gate_kl_wave_kernel<1>, gw, dim3(256), 0, st, a);
    else if (a.nb <= 512) hipLaunchKernelGGL(gate_kl_wave_kernel<2>, gw, dim3(256), 0, st, a);
    else if (a.nb <= 1024) hipLaunchKernelGGL(gate_kl_wave_kernel<4>, gw, dim3(256), 0, st, a);
    else if (a.nb <= 2048) hipLaunchKernelGGL(gate_kl_wave_kernel<8>, gw, dim3(256), 0, st, a);
    else if (a.nb <= 4096) hipLaunchKernelGGL(gate_kl_wave_kernel<16>, gw, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(gate_kl_kernel, dim3(a.nb, a.B * a.Hq), dim3(kST), 0, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nq = a.B * a.Hq;
  dim3 gd((a.nb + kBM - 1) / kBM, (a.Dg + kBN - 1) / kBN, 2 * nq);
  hipLaunchKernelGGL(gate_dproj_kernel, gd, dim3(kGT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.rope_base > 0.0) {
    if ((e = launch_rope(a, a.dqg, nq, a.dkg, nq, -1.0, st)) != hipSuccess) return e;
  }
  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  dim3 gw((3 * a.D + kBM - 1) / kBM, (a.Dg + kBN - 1) / kBN, a.Hq + hwk);
  hipLaunchKernelGGL(gate_dweight_kernel, gw, dim3(kGT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(gate_loss_kernel, dim3(1), dim3(kLossThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace seer
