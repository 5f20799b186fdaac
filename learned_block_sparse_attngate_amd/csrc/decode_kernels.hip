// Decode-stage block-sparse attention for gfx950: one query per head (the
// newest token) against the whole key/value cache, reading only the 64-token
// blocks the decode gate selected.
//
// Method ("SeerAttention: Self-distilled Attention Gating for Efficient
// Long-context Prefilling", responses on decoding): the decode gate picks the
// key blocks each query head needs, and only those blocks' K and V are read;
// the gate is distilled against the attention map max-pooled along the
// sequence (1D), which the dense mode here also emits.
//
// Design for CDNA4: the work is bound by reading the selected K/V blocks
// (a few FLOP per byte), so it stays on the vector units and is organized for
// memory parallelism:
//  * one workgroup per (batch, KV head, key split): the query heads of a GQA
//    group are processed together, so a block that several of them select is
//    read once; a block no head of the group selects is never read (the
//    split's active blocks are compacted on chip first);
//  * the next active block's K and V are loaded into registers while the
//    current one is processed, so every workgroup keeps two blocks in flight;
//  * the key range is split so that B * Hkv * splits fills the GPU; each
//    split keeps an online softmax per head and writes an unnormalized
//    partial (sum of p v, running max, sum of p) that a small kernel merges;
//  * Q . K: a lane quad per key, each lane a quarter of the head dimension,
//    quad shuffles for the sums; P . V: a thread per (8 dims, key group) with
//    16-byte V loads, partial sums kept per thread and reduced once per split;
//  * softmax in the log2 domain (the query is pre-scaled by log2(e)/sqrt(D)).
#include "seer_device.h"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kThreadsDec = 256;
constexpr int kMaxSplitBlocks = 256;         // blocks per key split (on-chip active list)
constexpr int kMaxSplits = 1024;

template <int D, int G8>
__global__ __launch_bounds__(kThreadsDec) void decode_attn_kernel(DecodeAttnArgs a) {
  constexpr int DQ = D / 4;                  // Q . K: dims per lane (a lane quad per key)
  constexpr int NV = D / 8;                  // P . V: groups of 8 dims (one 16-byte load)
  constexpr int KG = kThreadsDec / NV;       // P . V: key groups
  constexpr int KPT = kBlock / KG;           // P . V: keys per thread
  constexpr int NW = kThreadsDec / kWave;
  __shared__ float qs[G8][D];                // queries of the group, scaled to log2 units
  __shared__ float ps[2][G8][kBlock];        // scores, then probabilities (double buffered by block)
  __shared__ float alpha_s[2][G8];
  __shared__ float m_s[G8], l_s[G8];
  __shared__ uint16_t list[kMaxSplitBlocks];
  __shared__ uint8_t list_act[kMaxSplitBlocks];
  __shared__ int wcnt[NW];
  __shared__ float red[NW][G8][D];

  const int split = blockIdx.x;
  const int zg = blockIdx.y;                 // b * Hkv + g
  const int b = zg / a.Hkv, g = zg - b * a.Hkv;
  const int G = a.group;                     // <= G8, the compiled bound
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h_base = b * a.Hq + g * G;       // first query head (b, g*G)
  const int j0 = split * a.bps, j1 = min(a.nb, j0 + a.bps);

  for (int i = tid; i < G * D; i += kThreadsDec) {
    const int h = i / D, d = i - h * D;
    qs[h][d] = bf16_to_f32(a.q[static_cast<size_t>(h_base + h) * D + d]) * a.scale_log2;
  }
  if (tid < G) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  // active list of this split: blocks that some head of the group selects
  int cnt;
  {
    const int j = j0 + tid;
    unsigned act = 0;
    if (j < j1)
      for (int h = 0; h < G; ++h)
        if (a.mask == nullptr || a.mask[static_cast<size_t>(h_base + h) * a.nb + j] != 0) act |= 1u << h;
    const int f = act != 0;
    const int inc = wave_inclusive_scan(f, lane);
    if (lane == kWave - 1) wcnt[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wave; ++w2) base += wcnt[w2];
    if (f) {
      list[base + inc - 1] = static_cast<uint16_t>(j - j0);
      list_act[base + inc - 1] = static_cast<uint8_t>(act);
    }
    cnt = 0;
    for (int w2 = 0; w2 < NW; ++w2) cnt += wcnt[w2];
    __syncthreads();
  }

  const uint16_t* kbase = a.k + static_cast<size_t>(zg) * a.S * D;
  const uint16_t* vbase = a.v + static_cast<size_t>(zg) * a.S * D;
  const int uq = tid >> 2, c = tid & 3;      // Q . K: key, dim quarter
  const int dg = tid % NV, kg = tid / NV;    // P . V: dim group, key group

  float acc[G8][8];
#pragma unroll
  for (int h = 0; h < G8; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  // K slice (key uq, dims c*DQ ..) and V rows (keys kg + KG*i, dims dg*8 ..) of list entry n
  auto load = [&](int n, uint4 (&kr)[DQ / 8], uint4 (&vr)[KPT]) {
    const int t0 = (j0 + list[n]) * kBlock;
    const int n_tok = min(kBlock, a.S - t0);
    const uint4* kp = reinterpret_cast<const uint4*>(kbase + (static_cast<size_t>(t0) + min(uq, n_tok - 1)) * D + c * DQ);
#pragma unroll
    for (int i = 0; i < DQ / 8; ++i) kr[i] = kp[i];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = kg + KG * i;
      vr[i] = *reinterpret_cast<const uint4*>(vbase + (static_cast<size_t>(t0) + min(u, n_tok - 1)) * D + dg * 8);
    }
  };

  auto process = [&](int n, const uint4 (&kr)[DQ / 8], const uint4 (&vr)[KPT]) {
    const int buf = n & 1;
    const unsigned act = list_act[n];
    const int t0 = (j0 + list[n]) * kBlock;
    const int n_tok = min(kBlock, a.S - t0);
    // Q . K for the active heads
    float kf[DQ];
#pragma unroll
    for (int i = 0; i < DQ / 8; ++i) {
      const uint32_t wv[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[8 * i + 2 * e] = __uint_as_float(wv[e] << 16);
        kf[8 * i + 2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
      }
    }
    for (int h = 0; h < G; ++h) {
      if (!(act >> h & 1u)) continue;        // uniform
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) dot = fmaf(kf[i], qs[h][c * DQ + i], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      if (c == 0) ps[buf][h][uq] = uq < n_tok ? dot : -INFINITY;
    }
    __syncthreads();
    // online softmax per head (wave w takes heads w, w + 4)
    for (int h = wave; h < G; h += NW) {
      if (!(act >> h & 1u)) continue;        // uniform per wave
      const float sv = ps[buf][h][lane];
      const float bmax = wave_max(sv);
      const float mold = m_s[h];
      const float mnew = fmaxf(mold, bmax);
      const float pe = __builtin_amdgcn_exp2f(sv - mnew);     // 0 for keys past the cache
      const float bsum = wave_sum(pe);
      ps[buf][h][lane] = pe;
      if (lane == 0) {
        const float al = __builtin_amdgcn_exp2f(mold - mnew);   // 0 on the first block
        alpha_s[buf][h] = al;
        l_s[h] = l_s[h] * al + bsum;
        m_s[h] = mnew;
        if (a.gt != nullptr) a.gt[static_cast<size_t>(h_base + h) * a.nb + j0 + list[n]] = bmax;   // raw, log2
      }
    }
    __syncthreads();
    // P . V: each V element read once for every head
    float vf[KPT][8];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t wv[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[i][2 * e] = __uint_as_float(wv[e] << 16);
        vf[i][2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int h = 0; h < G8; ++h) {
      if (h >= G || !(act >> h & 1u)) continue;
      const float al = alpha_s[buf][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= al;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const float p = ps[buf][h][kg + KG * i];   // 0 past the cache
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[i][e], acc[h][e]);
      }
    }
    // no barrier here: the next block writes the other ps / alpha buffer, and
    // the one after that comes after two more barriers
  };

  if (cnt > 0) {
    uint4 kA[DQ / 8], vA[KPT], kB[DQ / 8], vB[KPT];
    load(0, kA, vA);
    for (int n = 0; n < cnt; n += 2) {
      if (n + 1 < cnt) load(n + 1, kB, vB);
      process(n, kA, vA);
      if (n + 1 >= cnt) break;
      if (n + 2 < cnt) load(n + 2, kA, vA);
      process(n + 1, kB, vB);
    }
  }

  // ---- partial of this split: sum over the key groups, then (acc, max, sum) per head
#pragma unroll
  for (int h = 0; h < G8; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e];
#pragma unroll
      for (int o = NV; o < kWave; o <<= 1) x += __shfl_xor(x, o);   // key groups inside the wave
      acc[h][e] = x;
    }
  if (lane < NV) {
#pragma unroll
    for (int h = 0; h < G8; ++h)
      if (h < G)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][h][dg * 8 + e] = acc[h][e];
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreadsDec) {
    const int h = i / D, d = i - h * D;
    float t = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) t += red[w2][h][d];
    a.part[(static_cast<size_t>(h_base + h) * a.nsplit + split) * (D + 2) + d] = t;
  }
  if (tid < G) {
    float* pr = a.part + (static_cast<size_t>(h_base + tid) * a.nsplit + split) * (D + 2);
    pr[D] = m_s[tid];
    pr[D + 1] = l_s[tid];
  }
}

// Merge the key splits of one (batch, head): O = sum_s 2^(m_s - M) acc_s / L,
// L = sum_s 2^(m_s - M) l_s, LSE = (M + log2 L) ln 2; in dense mode the raw
// block maxima become the 1D max-pooled map gt_j = 2^(r_j - log2-sum-exp).
// 1024 threads per row, so that the row takes few memory round trips: thread
// s reads split s's (max, sum) (splits <= kMaxSplits), then thread (part, d)
// sums dim d over splits part, part + P, ... with 8 loads in flight.
constexpr int kThreadsComb = 1024;
template <int D>
__global__ __launch_bounds__(kThreadsComb) void decode_combine_kernel(DecodeAttnArgs a) {
  constexpr int P = kThreadsComb / D;
  constexpr int NW = kThreadsComb / kWave;
  __shared__ float w_s[kMaxSplits];
  __shared__ float red[NW];
  __shared__ float o_s[P][D];
  const int z = blockIdx.x;                  // b * Hq + h
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* pp = a.part + static_cast<size_t>(z) * a.nsplit * (D + 2);
  const bool has = tid < a.nsplit;
  const float ms = has ? pp[static_cast<size_t>(tid) * (D + 2) + D] : -INFINITY;
  const float lsp = has ? pp[static_cast<size_t>(tid) * (D + 2) + D + 1] : 0.f;
  float mx = wave_max(ms);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  const float wt = (M > -INFINITY && ms > -INFINITY) ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
  if (has) w_s[tid] = wt;
  const float ls = wave_sum(lsp * wt);
  if (lane == 0) red[wave] = ls;
  __syncthreads();
  float L = 0.f;
  for (int w = 0; w < NW; ++w) L += red[w];
  const int d = tid % D, part = tid / D;
  float o8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // independent sums: many loads in flight
  int s = part;
  for (; s + 7 * P < a.nsplit; s += 8 * P)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o8[e] = fmaf(pp[static_cast<size_t>(s + e * P) * (D + 2) + d], w_s[s + e * P], o8[e]);
  for (; s < a.nsplit; s += P) o8[0] = fmaf(pp[static_cast<size_t>(s) * (D + 2) + d], w_s[s], o8[0]);
  o_s[part][d] = ((o8[0] + o8[1]) + (o8[2] + o8[3])) + ((o8[4] + o8[5]) + (o8[6] + o8[7]));
  __syncthreads();
  const float lse2 = L > 0.f ? M + __log2f(L) : -INFINITY;
  if (tid < D) {
    float t = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < P; ++p2) t += o_s[p2][tid];
    const float res = L > 0.f ? t / L : 0.f;
    if (a.out_bf16) {
      const uint32_t pk = pack_bf16x2(res, 0.f);
      static_cast<uint16_t*>(a.out)[static_cast<size_t>(z) * D + tid] = static_cast<uint16_t>(pk & 0xffffu);
    } else {
      static_cast<float*>(a.out)[static_cast<size_t>(z) * D + tid] = res;
    }
    if (tid == 0 && a.lse != nullptr) a.lse[z] = lse2 * 0.69314718055994530942f;
  }
  if (a.gt != nullptr)
    for (int j = tid; j < a.nb; j += kThreadsComb) {
      float* gp = a.gt + static_cast<size_t>(z) * a.nb + j;
      *gp = L > 0.f ? __builtin_amdgcn_exp2f(*gp - lse2) : 0.f;
    }
}

}  // namespace

// Key splits: about 512 (batch, KV head, split) workgroups, 8 to 256 blocks
// per split, at most 1024 splits. At 128k (8 KV heads, 2048 blocks) 512
// workgroups of 32 blocks measured 47 us against 50 us for 1024 of 16 and
// 59 us for 2048 of 8: fewer, longer splits pay the per-split setup less often.
void decode_split(int B, int Hkv, int nb, int* nsplit, int* bps) {
  const long long groups = static_cast<long long>(B) * Hkv;
  long long target = groups > 0 ? (512 + groups - 1) / groups : 1;
  if (target < 1) target = 1;
  long long per = (nb + target - 1) / target;
  if (per < 8) per = 8;
  if (per < (nb + kMaxSplits - 1) / kMaxSplits) per = (nb + kMaxSplits - 1) / kMaxSplits;
  if (per > kMaxSplitBlocks) per = kMaxSplitBlocks;
  *bps = static_cast<int>(per);
  *nsplit = nb > 0 ? static_cast<int>((nb + per - 1) / per) : 1;
}

template <int D>
void launch_decode_attn_d(const DecodeAttnArgs& a, dim3 grid, hipStream_t st) {
  // register arrays sized by the smallest compiled group bound that fits
  if (a.group <= 1) hipLaunchKernelGGL((decode_attn_kernel<D, 1>), grid, dim3(kThreadsDec), 0, st, a);
  else if (a.group <= 2) hipLaunchKernelGGL((decode_attn_kernel<D, 2>), grid, dim3(kThreadsDec), 0, st, a);
  else if (a.group <= 4) hipLaunchKernelGGL((decode_attn_kernel<D, 4>), grid, dim3(kThreadsDec), 0, st, a);
  else hipLaunchKernelGGL((decode_attn_kernel<D, kDecodeMaxGroup>), grid, dim3(kThreadsDec), 0, st, a);
}

hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t st) {
  const dim3 grid(a.nsplit, a.B * a.Hkv);
  if (a.D == 64) launch_decode_attn_d<64>(a, grid, st);
  else launch_decode_attn_d<128>(a, grid, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.D == 64) hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(a.B * a.Hq), dim3(kThreadsComb), 0, st, a);
  else hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(a.B * a.Hq), dim3(kThreadsComb), 0, st, a);
  return hipGetLastError();
}

}  // namespace seer
