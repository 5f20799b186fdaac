// Causal GQA block-sparse / dense FlashAttention-style forward for gfx950,
// plus the dense variant that records per-tile row maxima for the
// 2D-maxpooled ground truth.
//
// Method ("SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
// explainer section 3.4): the attention map is cut into 64 x 64 tiles aligned
// with the gate's blocks; a tile whose block-mask entry is 0 is skipped whole
// (no QK^T, no softmax, no PV and no K/V loads), a tile whose entry is 1 is
// processed with the FlashAttention-2 online softmax. For the ground truth
// (same page, "Training Procedure", customized training kernel) the kernel
// stores r = rowmax(S_ij) per query row and key tile, and after the row is
// finished rescales it with the final statistics (exp(r - m) / l) and takes a
// column max over the query block.
//
// Design for CDNA4:
//  * one workgroup = one (batch, query head, query block) row = 64 queries,
//    2 wavefronts x 32 queries; Q stays in registers for the whole row;
//  * both contractions use v_mfma_f32_32x32x16_bf16 with the matrix roles
//    chosen so the softmax is lane-local: S^T = K Q^T puts one query per lane
//    (32 of its keys in the lane, the other 32 in lane l^32), and
//    O^T = V^T P^T consumes the S^T registers directly as the B operand, so P
//    never goes through LDS;
//  * K and V tiles are staged through LDS with XOR swizzles that keep the
//    16-byte MFMA operand reads conflict-free; V is transposed in registers on
//    its way into LDS (keys permuted so each lane reads one 16-byte chunk);
//  * the next tile is fetched from HBM into registers while the current one is
//    computed;
//  * the active key blocks of a row are compacted on chip from the mask row
//    into an LDS list (ascending), so masked tiles cost neither time nor HBM
//    traffic and no separate compaction launch or workspace is needed;
//  * rows are launched heaviest first (descending query block) and, when the
//    head count allows, the query heads of one KV head are kept on one XCD so
//    that they share K/V tiles in that XCD's L2.
#include "seer_device.h"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kThreads = 128;          // 2 wavefronts
constexpr int kListCap = 2048;         // mask columns compacted per pass
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag by

enum Mode { kSparse = 0, kDense = 1, kDenseGt = 2 };

// Position <-> key permutation inside each 16-key group of a V^T row: swap
// bits 2 and 3. The 32x32 S^T accumulator gives lane half h the keys
// {8j + 4h + c}; storing V^T with this permutation lets that lane half fetch
// its 8 keys of a 16-key MFMA step as one contiguous 16-byte chunk.
__device__ __forceinline__ int key_of_pos(int p) {
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

// XOR swizzle of 16-byte chunks.
__device__ __forceinline__ int swz_k(int row) { return row & 7; }
__device__ __forceinline__ int swz_v(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ int bsum_exclusive(int x, int lane, int wave, int* wsum, int& total) {
  int inc = wave_inclusive_scan(x, lane);
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  int w0 = wsum[0];
  total = w0 + wsum[1];
  return inc - x + (wave == 1 ? w0 : 0);
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, D == 128 ? 1 : 2) void attn_fwd_kernel(AttnArgs p) {
  constexpr int CPR = D / 8;               // 16-byte chunks per K row
  constexpr int RG = kThreads / CPR;       // rows covered per load pass
  constexpr int RPT = kBlock / RG;         // K rows (V positions) per thread
  constexpr int KS = D / 16;               // MFMA k-steps for S^T
  constexpr int MT = D / 32;               // MFMA m-tiles for O^T

  __shared__ uint4 Ks[kBlock * CPR];       // K tile  [64 keys][D]   (swizzled chunks)
  __shared__ uint4 Vt[D * 8];              // V^T tile [D][64 keys]  (permuted, swizzled)
  __shared__ uint16_t list[MODE == kSparse ? kListCap : 1];
  __shared__ int wsum[2];
  __shared__ float lse_s[MODE == kDenseGt ? kBlock : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- which row: heaviest (last) query blocks first --------------------
  const int BH = p.B * p.Hq;
  const int w = blockIdx.x;
  const int qb = p.nb - 1 - w / BH;
  int local = w % BH;
  if (p.sched == 1) local = (local & 7) * (BH >> 3) + (local >> 3);  // heads of a KV group on one XCD
  const int bh = local;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.group;
  const size_t kv_off = (static_cast<size_t>(b) * p.Hkv + g) * p.S * D;
  const uint16_t* __restrict__ Kg = p.k + kv_off;
  const uint16_t* __restrict__ Vg = p.v + kv_off;

  // ---- Q fragment (B operand of S^T = K Q^T), resident for the row ------
  const int q_local = wave * 32 + l32;            // query row within the block
  const int t = qb * kBlock + q_local;            // query position
  const bool t_ok = t < p.S;
  uint4 qreg[KS];
  {
    const uint16_t* qrow = p.q + (static_cast<size_t>(bh) * p.S + (t_ok ? t : 0)) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = t_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * ks) : make_uint4(0, 0, 0, 0);
  }

  const float c = p.scale_log2;                   // log2(e) / sqrt(D)
  float m = -INFINITY;                            // running max (log2 units, may lag by kRescaleSlack)
  float lsum = 0.f;                               // this lane's partial row sum
  f32x16_t oacc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) oacc[i] = f32x16_t{};

  // load-thread geometry
  const int lc = tid % CPR;                       // 16-byte chunk (8 dims) this thread moves
  const int lr = tid / CPR;                       // row group

  uint4 kreg[RPT], vreg[RPT];
  auto fetch = [&](int kb) {
    const int key0 = kb * kBlock;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int kr = lr + RG * i;                 // K row in the tile
      const int kk = key0 + kr;
      kreg[i] = kk < p.S ? *reinterpret_cast<const uint4*>(Kg + static_cast<size_t>(kk) * D + 8 * lc)
                         : make_uint4(0, 0, 0, 0);
      const int vk = key0 + key_of_pos(RPT * lr + i);
      vreg[i] = vk < p.S ? *reinterpret_cast<const uint4*>(Vg + static_cast<size_t>(vk) * D + 8 * lc)
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int kr = lr + RG * i;
      Ks[kr * CPR + (lc ^ swz_k(kr))] = kreg[i];
    }
    // transpose 8 dims x RPT positions in registers, write RPT*2 bytes per dim
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int dim = 8 * lc + j;
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      uint32_t pk[RPT / 2];
#pragma unroll
      for (int pp = 0; pp < RPT / 2; ++pp) {
        const uint32_t lo = reinterpret_cast<const uint32_t*>(&vreg[2 * pp])[j >> 1];
        const uint32_t hi = reinterpret_cast<const uint32_t*>(&vreg[2 * pp + 1])[j >> 1];
        pk[pp] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      if constexpr (RPT == 8) {
        Vt[dim * 8 + (lr ^ swz_v(dim))] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      } else {  // RPT == 4: half a chunk
        uint2* dst = reinterpret_cast<uint2*>(&Vt[dim * 8 + ((lr >> 1) ^ swz_v(dim))]) + (lr & 1);
        *dst = make_uint2(pk[0], pk[1]);
      }
    }
  };

  const long long ntri_off = static_cast<long long>(qb) * (qb + 1) / 2;  // ground-truth scratch offset of this row
  auto compute = [&](int kb) {
    // S^T = K Q^T  (32 keys x 32 queries per m-tile, two m-tiles)
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int key = 32 * mt + l32;
        const uint4 a = Ks[key * CPR + ((2 * ks + hl) ^ swz_k(key))];
        sacc[mt] = mfma_32x32x16(a, qreg[ks], sacc[mt]);
      }
    }
    // element causality on the diagonal tile; row max
    const bool diag = (kb == qb);
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = sacc[mt][r];
        if (diag) {
          const int key = 32 * mt + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key > q_local) s = -INFINITY;
        }
        sacc[mt][r] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = pair_max(mx) * c;                         // row max of this tile, log2 units
    if constexpr (MODE == kDenseGt) {
      if (hl == 0)
        p.rmax[((static_cast<size_t>(bh) * p.ntri + ntri_off + kb) << 6) + q_local] = mx;
    }
    // lazy rescale: move the running max only when it grows by > slack
    const bool upd = mx > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float mn = upd ? mx : m;
      const float alpha = exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < MT; ++i) oacc[i] *= alpha;
      m = mn;
    }
    // P = exp2(s*c - m), packed to bf16 in the B-operand layout of O^T = V^T P^T
    uint4 pb[4];
    float ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float e[8];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          e[s8] = exp2f(fmaf(sacc[mt][8 * hh + s8], c, -m));
          ls += e[s8];
        }
        pb[2 * mt + hh] = make_uint4(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                     pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7]));
      }
    }
    lsum += ls;
    // O^T += V^T P^T  (32 dims x 32 queries per m-tile, 4 k-steps of 16 keys)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int dim = 32 * mt + l32;
        const uint4 a = Vt[dim * 8 + ((2 * ks + hl) ^ swz_v(dim))];
        oacc[mt] = mfma_32x32x16(a, pb[ks], oacc[mt]);
      }
    }
  };

  // ---- main loop over active key blocks -----------------------------------
  if constexpr (MODE == kSparse) {
    const uint8_t* mrow = p.mask + (static_cast<size_t>(bh) * p.nb + qb) * p.nb;
    const int ncol = qb + 1;                    // causal candidates 0..qb
    for (int c0 = 0; c0 < ncol; c0 += kListCap) {
      const int c1 = min(ncol, c0 + kListCap);
      // compaction: thread owns 16 consecutive columns
      const int j0 = c0 + 16 * tid;
      uint32_t bits = 0;
      if (j0 < c1) {
        if (j0 + 16 <= c1 && ((reinterpret_cast<uintptr_t>(mrow + j0) & 15) == 0)) {
          const uint4 v4 = *reinterpret_cast<const uint4*>(mrow + j0);
          const uint32_t wv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if ((wv[e >> 2] >> (8 * (e & 3))) & 0xffu) bits |= 1u << e;
        } else {
          for (int e = 0; e < 16 && j0 + e < c1; ++e)
            if (mrow[j0 + e]) bits |= 1u << e;
        }
      }
      int cnt_total;
      int pos = bsum_exclusive(__builtin_popcount(bits), lane, wave, wsum, cnt_total);
      while (bits) {
        const int e = __builtin_ctz(bits);
        bits &= bits - 1;
        list[pos++] = static_cast<uint16_t>(j0 + e);
      }
      __syncthreads();
      if (cnt_total > 0) {
        fetch(list[0]);
        for (int n = 0; n < cnt_total; ++n) {
          const int kb = list[n];
          __syncthreads();
          stage();
          __syncthreads();
          if (n + 1 < cnt_total) fetch(list[n + 1]);
          compute(kb);
        }
      }
      __syncthreads();                            // list and wsum reused by the next pass
    }
  } else {
    fetch(0);
    for (int kb = 0; kb <= qb; ++kb) {
      __syncthreads();
      stage();
      __syncthreads();
      if (kb < qb) fetch(kb + 1);
      compute(kb);
    }
  }

  // ---- epilogue: normalize, store O and LSE --------------------------------
  const float ltot = pair_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const float lse2 = ltot > 0.f ? m + __log2f(ltot) : -INFINITY;
  if (t_ok) {
    const size_t obase = (static_cast<size_t>(bh) * p.S + t) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = 32 * mt + 8 * r4 + 4 * hl;
        const float o0 = oacc[mt][4 * r4 + 0] * inv, o1 = oacc[mt][4 * r4 + 1] * inv;
        const float o2 = oacc[mt][4 * r4 + 2] * inv, o3 = oacc[mt][4 * r4 + 3] * inv;
        if (p.out_bf16) {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + dim) =
              make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + dim) = make_float4(o0, o1, o2, o3);
        }
      }
    }
    if (p.lse != nullptr && hl == 0) p.lse[static_cast<size_t>(bh) * p.S + t] = lse2 * kLn2;
  }

  if constexpr (MODE == kDenseGt) {
    // gt[qb, kb] = max over the block's queries of exp2(r - lse2); 0 above the diagonal
    if (hl == 0) lse_s[q_local] = t_ok ? lse2 : INFINITY;
    __syncthreads();                              // lse_s and this row's r writes visible to the workgroup
    float* gtrow = p.gt + (static_cast<size_t>(bh) * p.nb + qb) * p.nb;
    for (int kb = tid; kb < p.nb; kb += kThreads) {
      float best = 0.f;
      if (kb <= qb) {
        const float4* rr = reinterpret_cast<const float4*>(
            p.rmax + ((static_cast<size_t>(bh) * p.ntri + ntri_off + kb) << 6));
#pragma unroll 4
        for (int q4 = 0; q4 < 16; ++q4) {
          const float4 v = rr[q4];
          best = fmaxf(best, exp2f(v.x - lse_s[4 * q4 + 0]));
          best = fmaxf(best, exp2f(v.y - lse_s[4 * q4 + 1]));
          best = fmaxf(best, exp2f(v.z - lse_s[4 * q4 + 2]));
          best = fmaxf(best, exp2f(v.w - lse_s[4 * q4 + 3]));
        }
      }
      gtrow[kb] = best;
    }
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int mode, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B) * a.Hq * a.nb), block(kThreads);
  switch (mode) {
    case kSparse: hipLaunchKernelGGL((attn_fwd_kernel<D, kSparse>), grid, block, 0, st, a); break;
    case kDense: hipLaunchKernelGGL((attn_fwd_kernel<D, kDense>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((attn_fwd_kernel<D, kDenseGt>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int mode, hipStream_t st) {
  if (a.D == 64) return launch_d<64>(a, mode, st);
  return launch_d<128>(a, mode, st);
}

}  // namespace seer
