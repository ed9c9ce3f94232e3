// Internal definitions shared by the host planner and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sfa.h"

namespace sfa {

constexpr int kGranule = 16;       // token granule: finest bf16 row tiling of the MFMA
constexpr int kMaxFrameSlots = 1024;  // F + 1 limit (frame order table travels in kernel args)
constexpr int kMaxBlockGranules = 32;  // <= 512 query rows per item (16 tiles of 32)
constexpr int kNormChunk = 64;     // tokens per block in the norm kernels

// Visible key ranges of one query frame: [0, r0_end) and [r1_begin, r1_end)
// (r1 empty when the window touches frame 1 and the ranges merge).
struct KeyRanges {
  int32_t r0_end;
  int32_t r1_begin;
  int32_t r1_end;
};

// Key ranges of a set of frames made of the reference frame (if `ref`) and the
// contiguous window frames [lo, hi] (none if lo > hi), in the form above: range 0
// starts at token 0 (empty when the set lacks the reference frame), range 1 is the
// rest.
__host__ __device__ inline KeyRanges frame_set_ranges(bool ref, int lo, int hi, int T) {
  KeyRanges r;
  const bool win = lo <= hi;
  if (ref && win && lo == 1) {
    r.r0_end = (hi + 1) * T;
    r.r1_begin = r.r1_end = r.r0_end;
  } else if (ref) {
    r.r0_end = T;
    r.r1_begin = win ? lo * T : T;
    r.r1_end = win ? (hi + 1) * T : T;
  } else {
    r.r0_end = 0;
    r.r1_begin = lo * T;
    r.r1_end = (hi + 1) * T;
  }
  return r;
}

__host__ __device__ inline KeyRanges key_ranges(int f, int F, int T, int w) {
  KeyRanges r;
  if (f == 0) {
    r.r0_end = T;
    r.r1_begin = T;
    r.r1_end = T;
    return r;
  }
  const int lo = f - w > 1 ? f - w : 1;
  const int hi = f + w < F ? f + w : F;
  if (lo == 1) {
    r.r0_end = (hi + 1) * T;
    r.r1_begin = r.r0_end;
    r.r1_end = r.r0_end;
  } else {
    r.r0_end = T;
    r.r1_begin = lo * T;
    r.r1_end = (hi + 1) * T;
  }
  return r;
}

// Number of frames whose keys frame f sees (the cost of its work items).
__host__ __device__ inline int visible_frames(int f, int F, int w) {
  if (f == 0) return 1;
  const int lo = f - w > 1 ? f - w : 1;
  const int hi = f + w < F ? f + w : F;
  return 1 + (hi - lo + 1);
}

// Key split of a work item: the visible frames of query frame f (reference frame
// first, then the window in order) cut into two halves, the first holding the
// larger half. Each half is its own work item; the second of the two to finish adds
// the other's partial output and row sum to its own (exact for a shared fixed
// maximum, rescaled to the larger running maximum otherwise) and writes the result.
__host__ __device__ inline KeyRanges half_key_ranges(int f, int half, int F, int T, int w) {
  const int lo = f - w > 1 ? f - w : 1;
  const int hi = f + w < F ? f + w : F;
  const int n = 1 + (hi - lo + 1);  // visible frames: reference + window
  const int na = (n + 1) / 2;       // frames of the first half (reference + na - 1 window)
  if (half == 0) return frame_set_ranges(true, lo, lo + na - 2, T);
  return frame_set_ranges(false, lo + na - 1, hi, T);
}

// Entries of the plan's frame order: the query frame in bits 0-9, the key half + 1
// in bits 10-11 (0: whole item), the index of the split frame in bits 12-15.
constexpr int kMaxSplitFrames = 16;

struct Item {
  int32_t b, h, f, qb;
  int32_t half;   // -1: all visible keys; 0 / 1: the first / second half of them
  int32_t split;  // index of the split query frame (halves only)
};

// Item index -> work item. Groups of `nqb` items share one (frame, batch, head)
// key stream; groups are sorted by decreasing cost (frame_order). Item index i
// belongs to XCD i % 8 (the attention kernel's queues follow the round-robin
// order in which workgroups reach the XCDs), so inside every run of 8 groups the
// index is permuted to give each XCD one whole group (shared K/V in its L2)
// while the order still follows decreasing cost. The XCD -> group
// assignment rotates by one from run to run, so a head whose items are slower
// (online softmax) does not always land on the same XCD.
__host__ __device__ inline Item decode_item(int idx, const uint16_t* frame_order, int B, int H,
                                            int nqb, int items) {
  const int run = 8 * nqb;
  const int full = (items / run) * run;
  int logical = idx;
  if (idx < full) {
    const int c = idx / run;
    const int r = idx - c * run;
    logical = c * run + (((r & 7) + c) & 7) * nqb + (r >> 3);
  }
  const int g = logical / nqb;
  const int qb = logical - g * nqb;
  const int bh_count = B * H;
  const int fr = g / bh_count;
  const int bh = g - fr * bh_count;
  const int e = frame_order[fr];
  Item it;
  it.b = bh / H;
  it.h = bh - it.b * H;
  it.f = e & 1023;
  it.half = ((e >> 10) & 3) - 1;
  it.split = e >> 12;
  it.qb = qb;
  return it;
}

struct Workspace {
  size_t mu, kmax, qmax, bound, elig, kvis, fbound, felig, qn, qmu, psum, pkmax, pqmax, kst,
      vst, queue, part, split_cnt, total;
};

// Staged copies of K and V that the prologue writes for the attention kernel, in the
// layout its LDS stages use, so that every DMA request copies 1 KB of contiguous bytes
// and every MFMA operand read is a base register plus an immediate. Per (b, h) the
// tokens form 16-key granules of 32 * d bytes each:
//   K: [granule][16-byte chunk c of the d elements][16 keys]: element (key, e) of a
//      granule at (e / 8) * 128 + (key % 16) * 8 + e % 8;
//   V: [granule][d][16 keys], the two 16-byte halves of each d-row swapped when
//      (d / 8) is odd: element (key, e) at e * 16 + (((key / 8) ^ ((e / 8) & 1)) * 8)
//      + key % 8.
// Both are bf16, B * H * S * d elements, in (b, h)-major order.
__host__ __device__ constexpr int staged_granule_bytes(int d) { return 32 * d; }

// Partial result of one key half of a split item, in floats: O (not normalised) as
// [32-row query tile][32-dim tile][register][lane] for up to kPartRows rows, then the
// row sum l and the maximum m they are relative to, kPartRows rows each.
constexpr int kPartRows = 512;
// Counters per split item: one per pass over the keys (the online path of a kernel with
// two query tiles per wave makes one pass per tile).
constexpr int kSplitPasses = 2;
__host__ __device__ constexpr int part_floats(int d) {
  return kPartRows / 32 * (d / 32) * 16 * 64 + 2 * kPartRows;
}

// Work queue of the attention kernel in the workspace: one counter per XCD, a
// count of workgroups that found no work left, padding to 64 bytes.
constexpr int kQueueWords = 16;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t qsb, qss, qsh, ksb, kss, ksh, vsb, vss, vsh, osb, oss, osh;
  const float* qn;
  const float* qmu;
  const float* kvis;     // [b][h][F+1]: key-norm maximum the rows of each query frame use
  const uint8_t* felig;  // [b][h][F+1]: the items of the query frame take the fixed maximum
  const uint16_t* kst;   // K staged by the prologue (granule layout above)
  const uint16_t* vst;   // V staged by the prologue (granule layout above)
  int32_t B, H, S, T, F, w;
  int32_t gq;     // query granules per item (the last item of a frame: what is left)
  int32_t nqb;    // items per (frame, batch, head): ceil(T / (16 * gq))
  int32_t items;
  float c;        // scale * log2(e)
  int32_t* queue; // kQueueWords counters, zero between launches
  float* part;        // [split item][half] partial results (part_floats(d) each)
  int32_t* split_cnt; // [split item][pass]: halves finished, zero between launches
  uint16_t frame_order[kMaxFrameSlots];
};

struct NormParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t qsb, qss, qsh, ksb, kss, ksh, vsb, vss, vsh;
  uint16_t* kst;  // K and V staged for the attention kernels (granule layout above)
  uint16_t* vst;
  float* mu;
  float* kmax;
  float* qmax;
  float* bound;
  uint8_t* elig;
  float* kvis;    // [b][h][F+1]
  float* fbound;  // [b][h][F+1]
  uint8_t* felig; // [b][h][F+1]
  float* qn;
  float* qmu;
  float* psum;
  float* pkmax;   // [b][h][granule]: max ||k - mu||^2 over the 16 tokens of a granule
  float* pqmax;   // [b][h][granule]: max ||q||^2
  int32_t* queue; // the attention kernel's work queue, zeroed here
  int32_t* split_cnt;  // the split items' counters, zeroed here
  int32_t nsplit_cnt;
  int32_t B, H, S, D, nchunk;
  int32_t T, F, w;
  int32_t bound_mode;
  float scale;
  float bound_limit;
};

constexpr int kGenericBq = 256;  // ablation: query rows per block (8 waves x 32)
constexpr int kGenericBk = 128;  // ablation: keys per block (2 LDS stages of 64)

struct GenericParams {
  const uint16_t* q;
  const uint16_t* k;
  int64_t qsb, qss, qsh, ksb, kss, ksh;
  const uint16_t* kst;    // K and V staged (granule layout above)
  const uint16_t* vst;
  const int32_t* lists;   // key blocks: kb | (full << 30), per (pass, query block)
  const int32_t* offs;    // [2][nqb + 1] offsets into lists
  float* part;            // [2][b][h][S][d] per-pass normalised outputs
  float* lse;             // [2][b][h][S] per-pass log2-sum-exp2 of scale*log2(e)*s
  int32_t B, H, S, T, F, w, nqb, items;
  float c;                // scale * log2(e)
};

struct MergeParams {
  const float* part;
  const float* lse;
  uint16_t* o;
  int64_t osb, oss, osh;
  int32_t B, H, S, D;
};

// Fused prologue: D[feature][token] = W'[feature][:] . x[token][:] on 256 x 256
// workgroup tiles, scaled by the token's inverse RMS, rotated (q, k) and stored
// into q, k, v [b][s][h][e].
constexpr int kProTile = 256;   // features and tokens per workgroup tile
constexpr int kProKStage = 64;  // model-width elements per LDS stage

struct ProParams {
  const uint16_t* x;      // [b][s][C], C contiguous
  int64_t xsb, xss;       // element strides
  const uint16_t* w;      // W' = gamma * W, [3*H*d][C] bf16
  const float* cosv;      // [S][d/2]
  const float* sinv;
  uint16_t* out[3];       // q, k, v
  int64_t osb[3], oss[3], osh[3];
  int32_t B, S, C, H, d;
  int32_t ntile_f;        // 3*H*d / 256
  int32_t ntile_t;        // ceil(S / 256) per batch
  float eps;
};

}  // namespace sfa

struct sfa_generic {
  sfa_geometry g;
  float scale;
  int32_t S, nqb, nkb;
  int64_t full_blocks, partial_blocks, computed_pairs;
  int32_t* lists;       // host copy, copied into the workspace on every call
  int32_t nlist;
  int32_t* offs;        // [2][nqb + 1]
  size_t ws_kst, ws_vst, ws_lists, ws_offs, ws_part, ws_lse, ws_total;
};

struct sfa_plan {
  sfa_geometry g;
  float scale;
  int32_t S;
  int32_t gq;       // query granules per item (block_q / 16)
  int32_t waves;    // waves per attention workgroup (4 or 8)
  int32_t qt;       // 32-row query tiles per wave (1 or 2)
  int32_t stages;   // 64-key LDS stages in flight (2..4)
  int32_t nqb;      // ceil(T / block_q)
  int32_t bound_mode;  // 0: per-head key-norm maximum; 1: per visible frame
  int32_t items;
  int32_t nchunk;   // norm-kernel token chunks
  int32_t nslots;   // entries of frame_order: query frames, split ones twice
  int32_t nsplit;   // query frames whose items are split into two key halves
  int64_t active_pairs;
  sfa::Workspace ws;
  uint16_t frame_order[sfa::kMaxFrameSlots];
};

// Launchers (sfa_norms.hip / sfa_fwd.hip); return a hipError_t.
hipError_t sfa_launch_norms(const sfa::NormParams& p, hipStream_t stream);
hipError_t sfa_launch_fwd(const sfa::FwdParams& p, int head_dim, int waves, int qt, int stages,
                          hipStream_t stream);
hipError_t sfa_launch_stage(const sfa::NormParams& p, hipStream_t stream);
hipError_t sfa_launch_fold(const uint16_t* w, const uint16_t* gamma, uint16_t* out, int rows,
                           int cols, hipStream_t stream);
hipError_t sfa_launch_prologue(const sfa::ProParams& p, hipStream_t stream);
hipError_t sfa_launch_generic(const sfa::GenericParams& p, const sfa::MergeParams& m,
                              int head_dim, hipStream_t stream);
