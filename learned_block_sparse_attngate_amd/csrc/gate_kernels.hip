// AttnGate forward for gfx950: block pooling, per-head projections, causal
// block-level softmax and the threshold / top-k block mask.
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
//  gate_gemm        fp32 LDS-tiled GEMM (64 x 64 tiles, 4 x 4 per thread),
//                   used for the two projections and for the causal tiles of
//                   the block logits Q' K'^T.
//  gate_softmax_mask one workgroup per score row: max / sum reductions, the
//                   normalized row, and either the threshold or an exact
//                   4-pass radix select for top-k (ties to the lower index).
#include <math.h>

#include "seer_device.h"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kPoolThreads = 256;

template <int D>
__global__ __launch_bounds__(kPoolThreads) void gate_pool_kernel(GateArgs a) {
  constexpr int CPR = D / 8;              // 16-byte chunks per token row
  constexpr int NRG = kPoolThreads / CPR; // row groups
  __shared__ float red[3][NRG][D];

  const int i = blockIdx.x;
  const int H = a.Hq + a.Hkv;
  const int b = blockIdx.y / H;
  const int hx = blockIdx.y - b * H;
  const bool isq = hx < a.Hq;
  const uint16_t* src = isq ? a.q + (static_cast<size_t>(b) * a.Hq + hx) * a.S * D
                            : a.k + (static_cast<size_t>(b) * a.Hkv + (hx - a.Hq)) * a.S * D;
  const int t0 = i * kBlock;
  const int n = min(kBlock, a.S - t0);
  const int tid = threadIdx.x;
  const int c = tid % CPR;
  const int rg = tid / CPR;

  float sum[8], mx[8], mn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { sum[e] = 0.f; mx[e] = -INFINITY; mn[e] = INFINITY; }
  for (int r = rg; r < n; r += NRG) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(t0 + r) * D + 8 * c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
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

// ---------------------------------------------------------------------------
// fp32 tiled GEMM: C[m][n] = alpha * sum_k A[m][k] * Bm(k, n)
//   Bm(k, n) = B[k*ldb + n] (B_T = false) or B[n*ldb + k] (B_T = true)
// ---------------------------------------------------------------------------
constexpr int kGT = 256;
constexpr int kBM = 64, kBN = 64, kBK = 16;

template <bool B_T>
__device__ __forceinline__ void gemm_tile(const float* __restrict__ A, int lda, const float* __restrict__ B,
                                          int ldb, float* __restrict__ C, int ldc, int M, int N, int K,
                                          int m0, int n0, float alpha, bool causal_only) {
  __shared__ float As[kBK][kBM + 4];
  __shared__ float Bs[kBK][kBN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += kBK) {
    // A tile 64 x 16 (stored transposed), B tile 16 x 64
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + kGT * e;         // 0..1023
      const int am = idx >> 4, ak = idx & 15;
      const int gm = m0 + am, gk = k0 + ak;
      As[ak][am] = (gm < M && gk < K) ? A[static_cast<size_t>(gm) * lda + gk] : 0.f;
      int bk, bn;
      if (B_T) { bn = idx >> 4; bk = idx & 15; } else { bk = idx >> 6; bn = idx & 63; }
      const int gn = n0 + bn, gk2 = k0 + bk;
      float bv = 0.f;
      if (gn < N && gk2 < K) bv = B_T ? B[static_cast<size_t>(gn) * ldb + gk2] : B[static_cast<size_t>(gk2) * ldb + gn];
      Bs[bk][bn] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn >= N || (causal_only && gn > gm)) continue;
      C[static_cast<size_t>(gm) * ldc + gn] = acc[i][j] * alpha;
    }
  }
}

// Projections. blockIdx.z: 0 .. B*Hq-1 are Q' (one per query head), the rest
// are K' (one per query head, or one per KV head).
__global__ __launch_bounds__(kGT) void gate_proj_kernel(GateArgs a) {
  const int nq = a.B * a.Hq;
  const int z = blockIdx.z;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
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

// Causal 64 x 64 tiles of the block logits z = Q' K'^T / sqrt(D).
__global__ __launch_bounds__(kGT) void gate_logits_kernel(GateArgs a) {
  // triangular decode of blockIdx.x -> (ti, tj), tj <= ti
  const int idx = blockIdx.x;
  int ti = static_cast<int>((sqrtf(8.0f * idx + 1.0f) - 1.0f) * 0.5f);
  while ((ti + 1) * (ti + 2) / 2 <= idx) ++ti;
  while (ti * (ti + 1) / 2 > idx) --ti;
  const int tj = idx - ti * (ti + 1) / 2;
  const int z = blockIdx.y;                  // b * Hq + h
  const int b = z / a.Hq, h = z % a.Hq;
  const int hk = a.wk_per_kv ? h / a.group : h;
  const int hwk = a.wk_per_kv ? a.Hkv : a.Hq;
  const float* Aq = a.qg + static_cast<size_t>(z) * a.nb * a.Dg;
  const float* Bk = a.kg + (static_cast<size_t>(b) * hwk + hk) * a.nb * a.Dg;
  float* C = a.scores + static_cast<size_t>(z) * a.nb * a.nb;
  gemm_tile<true>(Aq, a.Dg, Bk, a.Dg, C, a.nb, a.nb, a.nb, a.Dg, ti * kBM, tj * kBN, a.scale, true);
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

__global__ __launch_bounds__(kST) void gate_softmax_mask_kernel(GateArgs a, TopkTable tk) {
  extern __shared__ float row[];             // nb floats
  __shared__ float red[kST / kWave];
  __shared__ int hist[256];
  __shared__ int sel_state[2];
  __shared__ int scan_tmp[kST / kWave];

  const int i = blockIdx.x;
  const int z = blockIdx.y;                  // b * Hq + h
  const int h = z % a.Hq;
  const int tid = threadIdx.x;
  const int n = i + 1;                       // causal entries of this row
  float* srow = a.scores + (static_cast<size_t>(z) * a.nb + i) * a.nb;
  uint8_t* mrow = a.mask + (static_cast<size_t>(z) * a.nb + i) * a.nb;

  float mx = -INFINITY;
  for (int j = tid; j < n; j += kST) {
    const float v = srow[j];
    row[j] = v;
    mx = fmaxf(mx, v);
  }
  mx = block_reduce_max(mx, red);
  float sum = 0.f;
  for (int j = tid; j < n; j += kST) {
    const float e = expf(row[j] - mx);
    row[j] = e;
    sum += e;
  }
  sum = block_reduce_sum(sum, red);
  const float inv = 1.0f / sum;
  for (int j = tid; j < a.nb; j += kST) {
    float s = 0.f;
    if (j < n) {
      s = row[j] * inv;
      row[j] = s;
    }
    srow[j] = s;
  }
  __syncthreads();

  if (a.mode == 0) {
    for (int j = tid; j < a.nb; j += kST) mrow[j] = (j < n && row[j] > a.threshold) ? 1 : 0;
    return;
  }

  // ---- top-k --------------------------------------------------------------
  const int k = tk.k[h];
  if (k >= n) {
    for (int j = tid; j < a.nb; j += kST) mrow[j] = j < n ? 1 : 0;
    return;
  }
  // radix select of the k-th largest value (scores are >= 0, so their bit
  // patterns order like the values)
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
  for (int j = n + tid; j < a.nb; j += kST) mrow[j] = 0;
}

}  // namespace

hipError_t launch_gate(const GateArgs& a, const TopkTable& tk, hipStream_t st) {
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

  const int T = (a.nb + kBM - 1) / kBM;
  dim3 gl(T * (T + 1) / 2, a.B * a.Hq);
  hipLaunchKernelGGL(gate_logits_kernel, gl, dim3(kGT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  dim3 gs(a.nb, a.B * a.Hq);
  hipLaunchKernelGGL(gate_softmax_mask_kernel, gs, dim3(kST), static_cast<size_t>(a.nb) * sizeof(float), st, a, tk);
  return hipGetLastError();
}

}  // namespace seer
