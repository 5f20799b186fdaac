// Kernel argument blocks and launchers shared between the host API and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace seer {

struct AttnArgs {
  const uint16_t* q;   // bf16 [B,Hq,S,D]
  const uint16_t* k;   // bf16 [B,Hkv,S,D]
  const uint16_t* v;   // bf16 [B,Hkv,S,D]
  const uint8_t* mask; // u8 [B,Hq,nb,nb] (sparse mode only)
  void* out;           // [B,Hq,S,D] fp32 or bf16
  float* lse;          // fp32 [B,Hq,S] or null
  float* rmax;         // ground-truth scratch [B*Hq][nb(nb+1)/2][64] fp32 (log2 units)
  float* gt;           // fp32 [B,Hq,nb,nb]
  int B, Hq, Hkv, S, D, nb, group;
  long long hs;        // tokens between consecutive heads' rows of q/k/v/out/lse (S; the packed length for varlen)
  long long ntri;      // nb(nb+1)/2
  float scale_log2;    // log2(e) / sqrt(D)
  int out_bf16;
  int sched;           // workgroup order of the dense kernels, see attn_fwd_kernel
  // block-sparse mode: key-chunked work items
  int chunk;           // key blocks per chunk (C)
  int nchunk;          // chunks per sequence = ceil(nb / C)
  long long items_per_group;  // work items per (batch, KV group)
  float* part_o;       // [items][64][D] fp32 normalized partial outputs (rows spanning > 1 chunk)
  float* part_l;       // [items][64] fp32 partial log2-sum-exp ([slots][64] on the XCD-owned path)
  int rotate;          // block-sparse: walk each row's tiles in the XCD-phased circular order
  // block-sparse, XCD-owned key chunks (persistent workgroups)
  int xcd;             // 1: this path (chunk = 128 blocks)
  int njobs;           // (batch, KV group, chunk) jobs
  long long slots_per_head;   // partial-output slots per (batch, head)
  uint16_t* part_o16;  // [B*Hq*slots_per_head][D/16 groups][128 threads][8] bf16 normalized partials
  int* xcd_ctr;        // 8 per-XCD item counters (zeroed by the launch)
  // block-sparse rows of one item, short sequences: active causal tiles of the
  // heads each XCD would own in the XCD-major order (counted by a pre-pass);
  // nullptr: that order is not considered
  int* xcd_work;
  int rows;            // block-sparse: one-item rows in the persistent launch (attn_sparse_rows_kernel, xcd_ctr)
};

// mode: 0 block-sparse (mask), 1 dense causal, 2 dense causal + ground-truth maxima
hipError_t launch_attn(const AttnArgs& a, int mode, hipStream_t st);

// Sequences of a packed batch that run in one launch (see attn_varlen_kernel):
// sequence i has t.len[i] > 0 tokens from packed token t.tok[i], its rows are
// workgroups row_start[i] .. row_start[i+1]-1 (Hq * nb_i of them), its
// [Hq, nb_i, nb_i] block map starts at element map_off[i] and its
// ground-truth scratch at float rmax_off[i].
constexpr int kVarlenMaxSeqs = 64;
struct VarlenTable {
  int n;
  int row_start[kVarlenMaxSeqs + 1];
  int tok[kVarlenMaxSeqs];
  int len[kVarlenMaxSeqs];
  long long map_off[kVarlenMaxSeqs];
  long long rmax_off[kVarlenMaxSeqs];
};
hipError_t launch_attn_varlen(const AttnArgs& a, const VarlenTable& t, int mode, hipStream_t st);
// key blocks per sweep chunk on the one-item-per-row block-sparse path (rows up to 1024 blocks)
int varlen_chunk_blocks();

// Work plan of the block-sparse kernel for one shape: which path, key chunks,
// item / slot counts and the workspace it needs.
struct SparsePlan {
  int xcd;                    // XCD-owned key chunks with persistent workgroups
  int chunk, nchunk;
  int rotate;                 // circular sweep (rows cut into chunks, other path)
  long long items_per_group;  // other path: (row, chunk) items per (batch, KV group)
  int njobs;                  // XCD path: (batch, KV group, chunk) jobs
  long long slots_per_head;   // XCD path: partial slots per (batch, head)
  int xcd_rows;               // one-item rows: the XCD-major order is taken when the mask's work is balanced
  int rows;                   // one-item rows in a persistent launch with per-XCD queues and stealing
  size_t workspace_bytes;
};
SparsePlan sparse_plan(int B, int Hkv, int group, int nb, int D);

struct GateArgs {
  const uint16_t* q;   // bf16 [B,Hq,S,D]
  const uint16_t* k;   // bf16 [B,Hkv,S,D]
  const float* wq;     // [Hq,D,Dg]
  const float* wk;     // [Hwk,3D,Dg]
  float* qp;           // [B,Hq,nb,D]
  float* kp;           // [B,Hkv,nb,3D]
  float* qg;           // [B,Hq,nb,Dg]
  float* kg;           // [B,Hwk,nb,Dg]
  float* scores;       // [B,Hq,nb,nb] (caller's output or workspace)
  uint8_t* mask;       // [B,Hq,nb,nb]
  int skip_scores;     // 1: the caller wants only the mask; the probabilities are not written back
  int B, Hq, Hkv, S, D, nb, Dg, group;
  long long hs;        // tokens between consecutive heads' rows of q/k (S; the packed length for varlen)
  int wk_per_kv;       // 1: Hwk = Hkv, 0: Hwk = Hq
  float scale;         // 1/sqrt(D)
  int mode;            // 0 threshold, 1 top-k
  float threshold;
  double rope_base;    // base theta / 64 of the gate's block RoPE; 0 = no RoPE
  // distillation step
  const float* gt;     // [B,Hq,nb,nb] 2D-maxpooled map
  float* dqg;          // [B,Hq,nb,Dg] d loss / d Q' (rotated, then back-rotated in place)
  float* dkg;          // [B,Hq,nb,Dg] d loss / d K' per query head
  float* row_loss;     // [B*Hq*nb]
  float* loss;         // [1]
  float* grad_wq;      // [Hq,D,Dg]
  float* grad_wk;      // [Hwk,3D,Dg]
};

constexpr int kMaxTopkHeads = 256;
struct TopkTable {
  int k[kMaxTopkHeads];
};

hipError_t launch_gate(const GateArgs& a, const TopkTable& tk, hipStream_t st);

// A packed batch's gate in one launch per stage: up to kGateVarlenMaxSeqs
// sequences that are consecutive in the batch, each the batch-1 problem at its
// token offset. GateArgs then describes the run: q/k at its first token (hs =
// the packed length), B = 1, scores/mask at its first sequence's maps, and
// the qp/kp/qg/kg (and, without a scores output, logits) regions hold every
// sequence's part one after another. Prefix sums over the run's sequences:
constexpr int kGateTile = 64;               // row / column tile of the gate's projections and logits
constexpr int kGateVarlenMaxSeqs = 64;
constexpr int kGateVarlenMaxBlocks = 4096;  // rows a wavefront keeps in registers
struct GateVarlenTable {
  int n;
  int tokp[kGateVarlenMaxSeqs + 1];        // tokens
  int nbp[kGateVarlenMaxSeqs + 1];         // 64-token blocks (the intermediates' offsets, pool and RoPE grids)
  int pp[kGateVarlenMaxSeqs + 1];          // projection row tiles
  int lp[kGateVarlenMaxSeqs + 1];          // logit tile workgroups (causal tiles x Hq)
  long long mp[kGateVarlenMaxSeqs + 1];    // nb^2 (map offsets, times Hq)
};
hipError_t launch_gate_varlen(const GateArgs& a, const TopkTable& tk, const GateVarlenTable& t, int max_nb,
                              hipStream_t st);

// Decode-stage gate: compressed K cache and per-token gate.
struct DecodeGateArgs {
  const uint16_t* q;   // bf16 [B,Hq,D], one query per head
  const uint16_t* k;   // bf16 [B,Hkv,S,D] key cache
  const float* wk;     // [Hwk,3D,D]
  float* kcomp;        // [B,Hwk,kcomp_blocks,D] compressed (pooled, projected) keys
  float* scores;       // [B,Hq,nb] or null
  uint8_t* mask;       // [B,Hq,nb]
  int B, Hq, Hkv, S, D, nb, group;
  int wk_per_kv;       // 1: Hwk = Hkv, 0: Hwk = Hq
  int kcomp_blocks;    // block capacity (row stride) of kcomp
  int block_begin;     // first block to (re)compute in the compressed cache
  float scale;         // 1/sqrt(D)
  int mode;            // 0 threshold, 1 top-k
  float threshold;
};
hipError_t launch_decode_kcomp(const DecodeGateArgs& a, hipStream_t st);
hipError_t launch_decode_gate(const DecodeGateArgs& a, const TopkTable& tk, hipStream_t st);

// Decode attention: one query per head against the key/value cache, reading
// only the blocks some head of the KV group selects.
constexpr int kDecodeMaxGroup = 8;
struct DecodeAttnArgs {
  const uint16_t* q;   // bf16 [B,Hq,D]
  const uint16_t* k;   // bf16 [B,Hkv,S,D]
  const uint16_t* v;   // bf16 [B,Hkv,S,D]
  const uint8_t* mask; // [B,Hq,nb] or null (every block)
  void* out;           // [B,Hq,D] fp32 or bf16
  float* lse;          // [B,Hq] or null
  float* gt;           // [B,Hq,nb] 1D max-pooled map or null (dense mode only)
  float* part;         // [B*Hq][nsplit][D + 2] partial (acc, max, sum) per key split
  uint32_t* blist;     // [B*Hkv][nb] block | selecting heads << 16, compacted per KV group (sparse mode)
  int* bcount;         // [B*Hkv] entries of blist per KV group
  int B, Hq, Hkv, S, D, nb, group;
  int nsplit, bps;     // key splits and blocks per split
  int out_bf16;
  float scale_log2;    // log2(e) / sqrt(D)
};
hipError_t launch_decode_attn(const DecodeAttnArgs& a, hipStream_t st);
void decode_split(int B, int Hkv, int nb, int* nsplit, int* bps);
// bytes of the decode-attention workspace: partials, then the compacted block lists
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int nb, int D);
hipError_t launch_gate_distill(const GateArgs& a, hipStream_t st);

}  // namespace seer
