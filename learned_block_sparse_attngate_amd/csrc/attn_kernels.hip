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
//    2 wavefronts x 32 queries, two workgroups per SIMD so that one wave's
//    MFMA work overlaps the other's softmax; Q stays in registers;
//  * both contractions use v_mfma_f32_32x32x16_bf16 with the matrix roles
//    chosen so the softmax is lane-local: S^T = K Q^T puts one query per lane
//    (32 of its keys in the lane, the other 32 in lane l^32), and
//    O^T = V^T P^T consumes the S^T registers directly as the B operand, so P
//    never goes through LDS;
//  * K and V tiles move HBM -> LDS with global_load_lds_dwordx4 (no register
//    staging); the XOR swizzle is applied on the source side so the LDS image
//    is conflict-free for the 16-byte K operand reads and for the
//    ds_read_b64_tr_b16 transposing reads that build the V^T operand;
//  * each wave copies the tile's operands from LDS into registers, then the
//    single LDS buffer is released and the next tile's copy is issued, so the
//    HBM/L2 latency of tile n+1 overlaps the softmax and P.V of tile n;
//  * the active key blocks of a row are compacted on chip from the mask row
//    into an LDS list (ascending), so masked tiles cost neither time nor HBM
//    traffic and no separate compaction launch or workspace is needed;
//  * rows are launched heaviest first (descending query block) and, when the
//    head count allows, the query heads of one KV head are kept on one XCD so
//    that they share K/V tiles in that XCD's L2.
#include <type_traits>

#include "seer_device.h"
#include "seer_internal.h"

namespace seer {

namespace {

constexpr int kThreads = 128;          // 2 wavefronts
constexpr int kListCap = 2048;         // mask columns compacted per pass
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag by
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer resource, dword 3

enum Mode { kSparse = 0, kDense = 1, kDenseGt = 2 };

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// 16-byte-chunk XOR swizzles (chunk index within a row of the LDS tile).
//  K: the 32x32x16 A-operand read has 16 consecutive keys at one logical chunk.
//  V: a ds_read_b64_tr_b16 reads 8 consecutive keys x 4 consecutive chunks.
template <int D> __device__ __forceinline__ int swz_k(int row) { return row & (D / 8 - 1); }
template <int D> __device__ __forceinline__ int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * (row & 1); }

__device__ __forceinline__ int bsum_exclusive(int x, int lane, int wave, int* wsum, int& total) {
  int inc = wave_inclusive_scan(x, lane);
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  int w0 = wsum[0];
  total = w0 + wsum[1];
  return inc - x + (wave == 1 ? w0 : 0);
}

template <int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs p) {
  constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
  constexpr int KS = D / 16;               // MFMA k-steps for S^T
  constexpr int MT = D / 32;               // MFMA m-tiles for O^T
  constexpr int RPI = 64 / CPR;            // tile rows per global_load_lds instruction
  constexpr int NDMA = 32 / RPI;           // instructions per wave per operand (32 rows)

  __shared__ uint4 Ks[kBlock * CPR];       // K tile [64 keys][D], swizzled chunks
  __shared__ uint4 Vs[kBlock * CPR];       // V tile [64 keys][D], swizzled chunks
  __shared__ uint16_t list[MODE == kSparse ? kListCap : 1];
  __shared__ int wsum[2];
  __shared__ float lse_s[MODE == kDenseGt ? kBlock : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- which row ---------------------------------------------------------
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2); all orders below launch the heaviest rows (last query blocks) first.
  //  0: heads interleaved, all KV groups at once;
  //  1: the query heads of one KV group on one XCD;
  //  2: KV-group major: every XCD works on the same KV group at a time, so
  //     the K/V working set is one group (it stays in the Infinity Cache);
  //  3: KV-group major, then head major inside the group.
  const int BH = p.B * p.Hq;
  const int w = blockIdx.x;
  int qb, bh;
  if (p.sched >= 2) {
    const int R = p.group * p.nb;                 // rows per (batch, KV group)
    const int gi = w / R, r = w - gi * R;         // gi = b * Hkv + g
    int hig;
    if (p.sched == 2) { qb = p.nb - 1 - r / p.group; hig = r % p.group; }
    else { hig = r / p.nb; qb = p.nb - 1 - r % p.nb; }
    const int bb = gi / p.Hkv, gg = gi - bb * p.Hkv;
    bh = bb * p.Hq + gg * p.group + hig;
  } else {
    qb = p.nb - 1 - w / BH;
    int local = w % BH;
    if (p.sched == 1) local = (local & 7) * (BH >> 3) + (local >> 3);
    bh = local;
  }
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

  // ---- HBM -> LDS copy of one K/V tile; this wave moves rows 32w .. 32w+31 --
  // buffer_load_dwordx4 ... lds: instruction i, lane l writes LDS bytes
  // [1024 i + 16 l) of this wave's half: tile row r = 32w + RPI*i + l/CPR,
  // physical chunk l%CPR, holding logical chunk (l%CPR) ^ swz(r). With the
  // swizzles above the V chunk does not depend on i and the K chunk takes four
  // values, so a few per-lane byte offsets address every instruction. The
  // buffer resource starts at the tile and ends at the head's last row, so rows
  // past the sequence (ragged last tile) read as zeros: their scores are masked
  // by causality and their P is 0.
  uint32_t kofs[4], vofs;
  {
    const int r0 = 32 * wave + lane / CPR;                  // row for i = 0
    const int pc = lane % CPR;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = r0 + RPI * v;                             // swz_k(r) for i = v (mod 4)
      kofs[v] = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_k<D>(r)));
    }
    vofs = static_cast<uint32_t>(r0 * 2 * D + 16 * (pc ^ swz_v<D>(r0)));
  }
  auto issue_tile = [&](int kb) {
    const int key0 = kb * kBlock;
    const int nbytes = (p.S - key0) * 2 * D;
    const auto kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kg + static_cast<size_t>(key0) * D), 0,
                                                      nbytes, kBufferWord3);
    const auto vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vg + static_cast<size_t>(key0) * D), 0,
                                                      nbytes, kBufferWord3);
    char* kl = reinterpret_cast<char*>(Ks) + 32 * wave * D * 2;
    char* vl = reinterpret_cast<char*>(Vs) + 32 * wave * D * 2;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const uint32_t step = static_cast<uint32_t>(RPI * i * 2 * D);
      const uint32_t ko = (D == 128 ? kofs[i & 3] : kofs[0]) + step;  // D = 64: swz_k(r) = r & 7 is i-invariant
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void_t*)(kl + 1024 * i), 16, ko, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void_t*)(vl + 1024 * i), 16, vofs + step, 0, 0, 0);
    }
  };

  const long long ntri_off = static_cast<long long>(qb) * (qb + 1) / 2;  // ground-truth scratch offset of this row

  // One tile. On entry the tile is in LDS (this wave's copy completed and the
  // workgroup synchronized); `next` >= 0 is issued as soon as both waves have
  // pulled their operands out of LDS.
  auto compute = [&](auto diag_tag, int kb, int next) {
    constexpr bool kDiag = decltype(diag_tag)::value;   // the diagonal tile needs element causality
    // operands of S^T = K Q^T: A = K rows (32 keys x 16 dims per m-tile / k-step)
    uint4 ka[2][KS];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int key = 32 * mt + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[mt][ks] = Ks[key * CPR + ((2 * ks + hl) ^ swz_k<D>(key))];
    }
    f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sacc[mt] = mfma_32x32x16(ka[mt][ks], qreg[ks], sacc[mt]);
    // keep the V^T reads below the S MFMAs so K and V operands are never live together
    __builtin_amdgcn_sched_barrier(0);

    // operands of O^T = V^T P^T: A = V^T (32 dims x 16 keys), two transposing
    // reads of 4 keys each; key order matches the S^T accumulator layout
    uint4 va[4][MT];
    {
      const int G = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          uint32_t half[4];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int key = 16 * ks + 8 * u + 4 * (G >> 1) + j;
            const int ch = 4 * mt + 2 * (G & 1) + (a >> 1);
            const int off = key * (2 * D) + ((ch ^ swz_v<D>(key)) << 4) + ((a & 1) << 3);
            const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(reinterpret_cast<char*>(Vs) + off));
            const uint2 r2 = __builtin_bit_cast(uint2, r);
            half[2 * u] = r2.x;
            half[2 * u + 1] = r2.y;
          }
          va[ks][mt] = make_uint4(half[0], half[1], half[2], half[3]);
        }
      }
    }

    // both waves hold their operands: release the buffer, start the next copy
    __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): all LDS reads returned
    __syncthreads();
    if (next >= 0) issue_tile(next);

    // element causality on the diagonal tile; row max
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (kDiag) {
          const int key = 32 * mt + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key > q_local) sacc[mt][r] = -INFINITY;
        }
        mx = fmaxf(mx, sacc[mt][r]);
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
      const float alpha = __builtin_amdgcn_exp2f(m - mn);   // m = -inf on the first tile: alpha = 0
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
          e[s8] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][8 * hh + s8], c, -m));
          ls += e[s8];
        }
        pb[2 * mt + hh] = make_uint4(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                     pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7]));
      }
    }
    lsum += ls;
    // O^T += V^T P^T  (32 dims x 32 queries per m-tile, 4 k-steps of 16 keys)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[mt] = mfma_32x32x16(va[ks][mt], pb[ks], oacc[mt]);
  };

  // wait for this wave's copy of the current tile, then make both halves visible
  auto tile_ready = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0f70);           // vmcnt(0)
    __syncthreads();
  };

  // ---- main loop over active key blocks -----------------------------------
  // The diagonal block (the only one needing element causality) goes first,
  // then the other active blocks in ascending order; dense rows use the same
  // order, so an all-ones mask reproduces the dense kernel bit for bit.
  if constexpr (MODE == kSparse) {
    const uint8_t* mrow = p.mask + (static_cast<size_t>(bh) * p.nb + qb) * p.nb;
    const bool diag_on = __builtin_amdgcn_readfirstlane(static_cast<int>(mrow[qb])) != 0;
    const int ncol = qb;                        // off-diagonal causal candidates 0..qb-1
    // compaction of columns [c0, c1): thread owns 16 consecutive columns
    auto compact = [&](int c0) {
      const int c1 = min(ncol, c0 + kListCap);
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
      return cnt_total;
    };
    int c0 = 0;
    int cnt = compact(0);
    bool issued = false;                        // list[0] of the current pass already in flight
    if (diag_on) {
      issue_tile(qb);
      tile_ready();
      const int first = cnt > 0 ? __builtin_amdgcn_readfirstlane(list[0]) : -1;
      compute(std::true_type{}, qb, first);
      issued = cnt > 0;
    }
    while (true) {
      if (cnt > 0) {
        int kb = __builtin_amdgcn_readfirstlane(list[0]);   // list entries are wave-uniform
        if (!issued) issue_tile(kb);
        for (int n = 0; n < cnt; ++n) {
          const int next = n + 1 < cnt ? __builtin_amdgcn_readfirstlane(list[n + 1]) : -1;
          tile_ready();
          compute(std::false_type{}, kb, next);
          kb = next;
        }
      }
      c0 += kListCap;
      if (c0 >= ncol) break;
      __syncthreads();                          // list and wsum are reused by the next pass
      cnt = compact(c0);
      issued = false;
    }
  } else {
    issue_tile(qb);
    tile_ready();
    compute(std::true_type{}, qb, qb > 0 ? 0 : -1);
    for (int kb = 0; kb < qb; ++kb) {
      tile_ready();
      compute(std::false_type{}, kb, kb + 1 < qb ? kb + 1 : -1);
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
