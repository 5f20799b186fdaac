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
// Design for CDNA4: the work is bound by reading the selected K/V blocks, so
// the arithmetic has to stay far below the memory time. It runs on the
// matrix cores with the prefill kernels' tile machinery:
//  * one wavefront per (batch, KV head, key split). The query heads of the
//    GQA group are the 32 columns of S^T = K Q^T (columns past the group are
//    zero), so a block that any head of the group selects is read once and
//    costs 32 MFMAs; a block no head selects is never read. A small kernel
//    first compacts each group's selected blocks into a list, and the splits
//    take even shares of it, so that no split reads many more blocks than
//    the others (a fixed block range per split left the splits that hold the
//    masks' stripes and sink several times the average);
//  * K and V tiles go HBM -> LDS with buffer_load ... lds in the prefill's
//    swizzled layout and are read with the same operand reads; P^T goes from
//    the S^T registers straight into O^T = V^T P^T. The wave owns its two
//    tile buffers, so the copy of block n+1's K starts as soon as block n's K
//    operands are in registers (V likewise) and no barrier is needed;
//  * each head (lane column) keeps an exact running max; keys past the cache
//    and heads that did not select a block get -inf scores (P = 0);
//  * the key range is split so that about kDecodeWaves wavefronts cover the
//    cache; each split writes an unnormalized partial (sum of p v, running
//    max, sum of p) per head, which a small kernel merges;
//  * softmax in the log2 domain (scores scaled by log2(e)/sqrt(D)).
#include "seer_device.h"
#include "seer_internal.h"
#include "tile_ops.h"

namespace seer {

namespace {

constexpr int kMaxSplitBlocks = 256;         // blocks per key split (on-chip active list)
constexpr int kMaxSplits = 1024;
constexpr int kDecodeWaves = 1024;           // split wavefronts per call, about (4 per CU)

template <int D>
__global__ __launch_bounds__(kWave) void decode_attn_kernel(DecodeAttnArgs a) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int KS = D / 16;                 // MFMA k-steps of S^T
  constexpr int MT = D / 32;                 // MFMA m-tiles of O^T
  constexpr int RPI = 64 / CPR;              // tile rows per copy instruction
  constexpr int NDMA = kBlock / RPI;         // copy instructions per tile and operand
  __shared__ uint4 Ks[kBlock * CPR];
  __shared__ uint4 Vs[kBlock * CPR];
  __shared__ uint32_t list[kMaxSplitBlocks]; // block - jbase | selecting heads << 16

  const int lane = threadIdx.x;
  const int l32 = lane & 31, hl = lane >> 5;
  const int split = blockIdx.x;
  const int zg = blockIdx.y;                 // b * Hkv + g
  const int b = zg / a.Hkv, g = zg - b * a.Hkv;
  const int G = a.group;                     // <= kDecodeMaxGroup
  const int h_base = b * a.Hq + g * G;       // first query head (b, g*G)
  const int j0 = split * a.bps, j1 = min(a.nb, j0 + a.bps);

  // active list of this split. Sparse mode: an even share of the KV group's
  // compacted list (blocks that some head of the group selects), so that
  // every split reads about as many blocks; dense mode: the block range.
  int cnt = 0;
  if (a.mask != nullptr) {
    const int total = a.bcount[zg];
    const int per = (total + a.nsplit - 1) / a.nsplit;    // <= bps
    const int e0 = min(total, split * per), e1 = min(total, e0 + per);
    const uint32_t* src = a.blist + static_cast<size_t>(zg) * a.nb;
    for (int e = e0 + lane; e < e1; e += kWave) list[e - e0] = src[e];   // absolute blocks
    cnt = e1 - e0;
  }
  const int jbase = a.mask != nullptr ? 0 : j0;  // list entries hold block - jbase
  for (int jb = j0; a.mask == nullptr && jb < j1; jb += kWave) {
    const int j = jb + lane;
    const uint32_t act = j < j1 ? (1u << G) - 1u : 0u;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(act != 0);
    if (act != 0) {
      const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u)));
      list[cnt + below] = static_cast<uint32_t>(j - j0) | (act << 16);
    }
    cnt += __popcll(bal);
  }
  // B operand of S^T = K Q^T: column l32 is query head h_base + l32 (zero past
  // the group), dims 16 ks + 8 hl .. +7
  const bool col = l32 < G;
  uint4 qreg[KS];
  {
    const uint16_t* qrow = a.q + static_cast<size_t>(h_base + (col ? l32 : 0)) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = col ? *reinterpret_cast<const uint4*>(qrow + 16 * ks) : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();                           // the list is in LDS
  wait_vm_le<0>();                           // and the Q rows in registers

  // copies of the tile at token t0 (rows past the cache read as zeros):
  // instruction i moves rows RPI i .. RPI i + RPI - 1, 1 KiB further on in
  // memory and in LDS; the immediate offset carries i % 4 (it holds 12 bits)
  uint32_t kofs[4], vofs;
  {
    const int r0 = lane / CPR, pc = lane % CPR;
#pragma unroll
    for (int u = 0; u < 4; ++u) kofs[u] = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_k<D>(r0 + RPI * u)));
    vofs = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_v<D>(r0)));
  }
  const uint16_t* kbase = a.k + static_cast<size_t>(zg) * a.S * D;
  const uint16_t* vbase = a.v + static_cast<size_t>(zg) * a.S * D;
  auto issue = [&](const uint16_t* base, uint4* buf, bool is_k, int t0) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + static_cast<size_t>(t0) * D), 0,
                                                      (a.S - t0) * 2 * D, kBufferWord3);
    char* dst = reinterpret_cast<char*>(buf);
    static_for<NDMA>([&](auto I) {
      constexpr int i = decltype(I)::value, hi = i / 4;
      const uint32_t ofs = is_k ? (D == 128 ? kofs[i & 3] : kofs[0]) : vofs;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + 4096 * hi), 16, ofs + 4096 * hi, 0,
                                               1024 * (i % 4), 0);
    });
  };
  uint32_t kaddr[KS], vaddr[MT];
  {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kaddr[ks] = lds_addr(Ks) + l32 * 2 * D + 16 * ((2 * ks + hl) ^ swz_k<D>(l32));
    const int G4 = lane >> 4, jj = (lane >> 2) & 3, aa = lane & 3;
    const int key = 4 * (G4 >> 1) + jj;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      vaddr[mt] = lds_addr(Vs) + key * 2 * D + 16 * ((4 * mt + 2 * (G4 & 1) + (aa >> 1)) ^ swz_v<D>(key)) + 8 * (aa & 1);
  }

  const float c = a.scale_log2;
  float m = -INFINITY, lsum = 0.f;
  f32x16_t oacc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) oacc[i] = f32x16_t{};

  if (cnt > 0) {
    // list entries are read with waits of their own, outside the compiler's
    // view of the copies in flight (it would otherwise wait for all of them),
    // and kept in scalar registers (the copies take a scalar base address)
    uint32_t e = __builtin_amdgcn_readfirstlane(lds_read_u32(lds_addr(&list[0])));
    int t0 = (jbase + static_cast<int>(e & 0xffffu)) * kBlock;
    issue(kbase, Ks, true, t0);
    issue(vbase, Vs, false, t0);
    const bool want_gt = a.gt != nullptr;
    const uint32_t all_heads = (1u << G) - 1u;
    for (int n = 0; n < cnt; ++n) {
      const uint32_t act = e >> 16;
      const int jcur = jbase + static_cast<int>(e & 0xffffu);
      const int tcur = t0;
      const bool more = n + 1 < cnt;
      if (more) {
        e = __builtin_amdgcn_readfirstlane(lds_read_u32(lds_addr(&list[n + 1])));
        t0 = (jbase + static_cast<int>(e & 0xffffu)) * kBlock;
      }
      // K of this block has landed once only its V copy (and the previous
      // block's map store) is younger
      if (want_gt && n > 0) wait_vm_le<NDMA + 1>();
      else wait_vm_le<NDMA>();
      u32x4_t kr[2 * KS];
      read_k_tile<D>(kaddr, kr);
      if (more) issue(kbase, Ks, true, t0);
      f32x16_t sacc[2];
      sacc[0] = f32x16_t{};
      sacc[1] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          sacc[mt] = mfma_32x32x16(__builtin_bit_cast(uint4, kr[2 * ks + mt]), qreg[ks], sacc[mt]);
      // -inf for keys past the cache and for heads that did not select the
      // block (columns past the group compute on zero queries and are never
      // stored); most blocks are whole and selected by every head
      const int n_tok = min(kBlock, a.S - tcur);
      const bool on = col && ((act >> l32) & 1u);
      if (n_tok < kBlock || act != all_heads) {
        // key 32 mt + 8 (r / 4) + 4 hl + r % 4 >= n_tok, with the lane's part on the right
        const int lim = on ? n_tok - 4 * hl : -kBlock;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * mt + 8 * (r >> 2) + (r & 3) >= lim) sacc[mt][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
      const float bmax = pair_max(mx) * c;   // block max of the head, log2 units
      // V of this block has landed once only the next block's K copy is younger
      if (more) wait_vm_le<NDMA>();
      else wait_vm_le<0>();
      u32x2_t vr[8 * MT];
      read_v_tile<D>(vaddr, vr);
      // the map store sits between this block's V wait and the next V copy,
      // which the next K wait counts; the map exists only in dense mode,
      // where lane 0 always stores, so it is exactly one store instruction
      if (want_gt && hl == 0 && on) a.gt[static_cast<size_t>(h_base + l32) * a.nb + jcur] = bmax;
      if (more) issue(vbase, Vs, false, t0);
      // online softmax (exact running max) and O^T += V^T P^T
      const float mn = fmaxf(m, bmax);
      if (__builtin_amdgcn_ballot_w64(mn > m)) {
        const float alpha = mn > m ? __builtin_amdgcn_exp2f(m - mn) : 1.f;   // m = -inf: 0
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < MT; ++i) oacc[i] *= alpha;
      }
      m = mn;
      const float mu = m == -INFINITY ? 0.f : m;   // no score yet: P = exp2(-inf) = 0
      uint4 pb[4];
      float ls = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float ev[8];
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) {
            ev[s8] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][8 * hh + s8], c, -mu));
            ls += ev[s8];
          }
          pb[2 * mt + hh] = make_uint4(pack_bf16x2(ev[0], ev[1]), pack_bf16x2(ev[2], ev[3]),
                                       pack_bf16x2(ev[4], ev[5]), pack_bf16x2(ev[6], ev[7]));
        }
      lsum += ls;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x2_t lo = vr[(ks * MT + mt) * 2], hi = vr[(ks * MT + mt) * 2 + 1];
          oacc[mt] = mfma_32x32x16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb[ks], oacc[mt]);
        }
    }
  }

  // partial of this split per head: O^T column l32, dims 32 mt + 8 r4 + 4 hl ..
  const float ltot = pair_sum(lsum);
  if (col) {
    float* pr = a.part + (static_cast<size_t>(h_base + l32) * a.nsplit + split) * (D + 2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * mt + 8 * r4 + 4 * hl;
        *reinterpret_cast<float2*>(pr + dim) = make_float2(oacc[mt][4 * r4 + 0], oacc[mt][4 * r4 + 1]);
        *reinterpret_cast<float2*>(pr + dim + 2) = make_float2(oacc[mt][4 * r4 + 2], oacc[mt][4 * r4 + 3]);
      }
    if (hl == 0) {
      pr[D] = m;
      pr[D + 1] = ltot;
    }
  }
}


// Compacted block list of each (batch, KV group) for sparse mode: the blocks
// that some head of the group selects, ascending, as block | heads << 16, and
// their count. One workgroup per group; 1024 blocks per round, ordered by a
// ballot inside each wavefront and the wavefront totals across them.
constexpr int kListThreads = 1024;
__global__ __launch_bounds__(kListThreads) void decode_list_kernel(DecodeAttnArgs a) {
  __shared__ int wsum[kListThreads / kWave];
  const int zg = blockIdx.x;
  const int b = zg / a.Hkv, g = zg - b * a.Hkv;
  const int G = a.group;
  const int h_base = b * a.Hq + g * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* dst = a.blist + static_cast<size_t>(zg) * a.nb;
  int base = 0;
  for (int jb = 0; jb < a.nb; jb += kListThreads) {
    const int j = jb + tid;
    uint32_t act = 0;
    if (j < a.nb)
      for (int h = 0; h < G; ++h)
        if (a.mask[static_cast<size_t>(h_base + h) * a.nb + j] != 0) act |= 1u << h;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(act != 0);
    const int below = static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u)));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int before = base, tot = 0;
    for (int w = 0; w < kListThreads / kWave; ++w) {
      if (w < wave) before += wsum[w];
      tot += wsum[w];
    }
    if (act != 0) dst[before + below] = static_cast<uint32_t>(j) | (act << 16);
    base += tot;
    __syncthreads();                         // wsum is rewritten next round
  }
  if (tid == 0) a.bcount[zg] = base;
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

// Key splits: about kDecodeWaves (batch, KV head, split) wavefronts, 8 to
// 256 blocks per split, at most kMaxSplits splits.
void decode_split(int B, int Hkv, int nb, int* nsplit, int* bps) {
  const long long groups = static_cast<long long>(B) * Hkv;
  long long target = groups > 0 ? (kDecodeWaves + groups - 1) / groups : 1;
  if (target < 1) target = 1;
  long long per = (nb + target - 1) / target;
  if (per < 8) per = 8;
  if (per < (nb + kMaxSplits - 1) / kMaxSplits) per = (nb + kMaxSplits - 1) / kMaxSplits;
  if (per > kMaxSplitBlocks) per = kMaxSplitBlocks;
  *bps = static_cast<int>(per);
  *nsplit = nb > 0 ? static_cast<int>((nb + per - 1) / per) : 1;
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int nb, int D) {
  int nsplit = 1, bps = 1;
  decode_split(B, Hkv, nb, &nsplit, &bps);
  const size_t part = static_cast<size_t>(B) * Hq * nsplit * (D + 2) * sizeof(float);
  return (part + 15) / 16 * 16 + static_cast<size_t>(B) * Hkv * (static_cast<size_t>(nb) + 1) * sizeof(uint32_t);
}

hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t st) {
  if (a.mask != nullptr) {
    hipLaunchKernelGGL(decode_list_kernel, dim3(a.B * a.Hkv), dim3(kListThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(a.nsplit, a.B * a.Hkv);
  if (a.D == 64) hipLaunchKernelGGL(decode_attn_kernel<64>, grid, dim3(kWave), 0, st, a);
  else hipLaunchKernelGGL(decode_attn_kernel<128>, grid, dim3(kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.D == 64) hipLaunchKernelGGL(decode_combine_kernel<64>, dim3(a.B * a.Hq), dim3(kThreadsComb), 0, st, a);
  else hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(a.B * a.Hq), dim3(kThreadsComb), 0, st, a);
  return hipGetLastError();
}

}  // namespace seer
