// C ABI: planning (host only), argument validation and kernel launches.
//
// Planning follows "HeyGen x Google Cloud: Bringing Avatar IV to TPUs",
// section "Deleting the mask": query blocks are whole 16-token granules inside
// one frame (the frame span T is a multiple of 16), so every (query block, key
// granule) pair is either fully visible or skipped and the key loop never needs
// a mask or padding.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "sfa_internal.h"

using namespace sfa;

// Workspace of sfa_attention_static: one copy on every GPU the library runs it on, held
// until the process ends. Host code never uses this name as an address: it asks the
// runtime for each device's copy (static_scratch below).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

thread_local hipError_t g_last_hip = hipSuccess;
thread_local char g_msg[256];

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SFA_OK;
  g_last_hip = e;
  return SFA_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// 126 / (2 * log2(e)): the largest eligibility threshold whose weights stay normal floats
constexpr float kMaxBoundLimit = 43.668f;

int validate_geometry(const sfa_geometry* g) {
  if (!g) return SFA_ERR_INVALID;
  if (g->batch < 1 || g->heads < 1 || g->frames < 0 || g->window < 0 ||
      g->tokens_per_frame < 1)
    return SFA_ERR_INVALID;
  if (!(g->scale >= 0.0f) || !isfinite(g->scale) || isnan(g->bound_limit))
    return SFA_ERR_INVALID;
  // a fixed maximum more than 2 * bound_limit above the largest logit would let the
  // largest weight of a row underflow: exp2(-2 * log2(e) * bound_limit) must stay a
  // normal float (>= 2^-126)
  if (g->bound_limit > kMaxBoundLimit) return SFA_ERR_UNSUPPORTED;
  if (g->head_dim != 64 && g->head_dim != 128) return SFA_ERR_UNSUPPORTED;
  if (g->tokens_per_frame % kGranule != 0) return SFA_ERR_UNSUPPORTED;
  if (g->frames + 1 > kMaxFrameSlots) return SFA_ERR_UNSUPPORTED;
  const int64_t S = int64_t(g->frames + 1) * g->tokens_per_frame;
  // 32-bit token and row indices inside the kernels; one head's V^T (d x S bf16)
  // is addressed with 32-bit byte offsets
  if (S * g->heads * int64_t(g->batch) > (int64_t(1) << 31) - 1) return SFA_ERR_UNSUPPORTED;
  if (S * g->head_dim * 2 > (int64_t(1) << 31) - 1) return SFA_ERR_UNSUPPORTED;
  return SFA_OK;
}

// Compute units the default block size aims to keep busy (MI355X: 256).
constexpr int kTargetItems = 256;

// Query granules per work item: as many as one workgroup holds (waves x query tiles
// of 32 rows), or the whole frame when it is shorter. The last block of a frame takes
// the remaining rows, so a frame costs ceil(T / 32) wave tiles, the fewest possible
// (a block size that divides T, such as 240 rows for T = 3600, leaves 16 repeated
// rows in the last wave tile of every block). When those blocks give fewer work items
// than compute units (small layers), each frame is cut into the most blocks that still
// give every compute unit at most one item, of balanced size, but not less than one
// wave's rows: a block's time falls less than its rows do (its keys stream at a rate
// of their own), so a second round of items costs more than larger blocks.
// slots = work items per query block index (batch x heads x frame slots, a split frame
// counting twice).
int auto_block_granules(int t_granules, int max_granules, int min_granules, int64_t slots) {
  const int top = t_granules < max_granules ? t_granules : max_granules;
  if (top <= min_granules) return top;
  if (slots * ((t_granules + top - 1) / top) >= kTargetItems) return top;
  const int64_t nqb = kTargetItems / slots;  // >= 1 here
  int64_t gq = (t_granules + nqb - 1) / nqb;
  if (gq < min_granules) gq = min_granules;
  return gq > top ? top : int(gq);
}

int create(const sfa_geometry* geom, const sfa_plan_options* opt, sfa_plan** out) {
  if (!out) return SFA_ERR_INVALID;
  *out = nullptr;
  int st = validate_geometry(geom);
  if (st != SFA_OK) return st;
  const int T = geom->tokens_per_frame;
  const int tg = T / kGranule;
  const int block_q = opt ? opt->block_q : 0;
  const int waves = (opt && opt->waves_per_item) ? opt->waves_per_item : 8;
  if (waves != 4 && waves != 8 && waves != 12) return SFA_ERR_UNSUPPORTED;
  const int wave_rows = (opt && opt->wave_rows) ? opt->wave_rows : (waves == 4 ? 64 : 32);
  if (wave_rows != 32 && wave_rows != 64) return SFA_ERR_UNSUPPORTED;
  if (waves == 4 && wave_rows != 64) return SFA_ERR_UNSUPPORTED;
  if (waves == 12 && wave_rows != 32) return SFA_ERR_UNSUPPORTED;
  const int qt = wave_rows / 32;
  const int max_granules = waves * wave_rows / kGranule;
  const int stages = (opt && opt->lds_stages) ? opt->lds_stages : 3;
  if (stages < 2 || stages > (waves == 12 ? 3 : 4)) return SFA_ERR_UNSUPPORTED;
  const int bound_mode = opt ? opt->bound_mode : 0;
  if (bound_mode != 0 && bound_mode != 1) return SFA_ERR_UNSUPPORTED;
  const int key_split = opt ? opt->key_split : 0;
  if (key_split != 0 && key_split != -1) return SFA_ERR_UNSUPPORTED;
  const int F = geom->frames, w = geom->window, B = geom->batch, H = geom->heads;
  // Key split of the tail: the items of the cheapest query frames that see more than
  // one frame are the last multi-frame items the largest-first order starts, and the
  // longest of the short items that end the launch; each is split into two key halves
  // (frames ordered reference first), so the tail is made of items half as long. Only
  // the kernels of 8 or 12 waves merge halves.
  int vmin = 0;
  if (key_split == 0 && waves >= 8)
    for (int f = 1; f <= F; ++f) {
      const int v = visible_frames(f, F, w);
      if (v >= 2 && (vmin == 0 || v < vmin)) vmin = v;
    }
  int nsplit = 0;
  if (vmin > 0)
    for (int f = 1; f <= F; ++f) nsplit += visible_frames(f, F, w) == vmin;
  if (nsplit > kMaxSplitFrames || F + 1 + nsplit > kMaxFrameSlots) nsplit = 0;
  int gq;
  if (block_q == 0) {
    gq = auto_block_granules(tg, max_granules, wave_rows / kGranule,
                             int64_t(B) * H * (F + 1 + nsplit));
  } else {
    if (block_q < 0 || block_q % kGranule != 0 || block_q / kGranule > max_granules)
      return SFA_ERR_UNSUPPORTED;
    gq = block_q / kGranule;
    if (gq > tg) gq = tg;  // one block holds the whole frame
  }
  sfa_plan* p = new (std::nothrow) sfa_plan;
  if (!p) return SFA_ERR_NOMEM;
  memset(p, 0, sizeof(*p));
  p->g = *geom;
  const int D = geom->head_dim;
  p->scale = geom->scale == 0.0f ? 1.0f / sqrtf(float(D)) : geom->scale;
  p->S = (F + 1) * T;
  p->gq = gq;
  p->waves = waves;
  p->qt = qt;
  p->stages = stages;
  p->bound_mode = bound_mode;
  p->nqb = (tg + gq - 1) / gq;  // the last block of a frame may be shorter
  p->nchunk = (p->S + kNormChunk - 1) / kNormChunk;

  // slots: every query frame once, a split one as two halves; by decreasing cost (number
  // of visible frames of the slot), ties in slot order
  int cost[kMaxFrameSlots];
  int ns = 0, si = 0;
  for (int f = 0; f <= F; ++f) {
    const int v = visible_frames(f, F, w);
    if (nsplit > 0 && f > 0 && v == vmin) {
      p->frame_order[ns] = uint16_t(f | (1 << 10) | (si << 12));
      cost[ns++] = (v + 1) / 2;
      p->frame_order[ns] = uint16_t(f | (2 << 10) | (si << 12));
      cost[ns++] = v / 2;
      ++si;
    } else {
      p->frame_order[ns] = uint16_t(f);
      cost[ns++] = v;
    }
  }
  int idx[kMaxFrameSlots];
  for (int i = 0; i < ns; ++i) idx[i] = i;
  std::stable_sort(idx, idx + ns, [&](int a, int b) { return cost[a] > cost[b]; });
  uint16_t sorted[kMaxFrameSlots];
  for (int i = 0; i < ns; ++i) sorted[i] = p->frame_order[idx[i]];
  memcpy(p->frame_order, sorted, sizeof(uint16_t) * ns);
  p->nslots = ns;
  p->nsplit = nsplit;
  p->items = B * H * ns * p->nqb;
  int64_t frame_pairs = 0;
  for (int f = 0; f <= F; ++f) frame_pairs += visible_frames(f, F, w);
  p->active_pairs = frame_pairs * int64_t(T) * T * B * H;

  // workspace layout (all fp32 unless noted), 256-byte aligned sections
  const size_t bh = size_t(B) * H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  p->ws.mu = take(bh * D * 4);
  p->ws.kmax = take(bh * 4);
  p->ws.qmax = take(bh * 4);
  p->ws.bound = take(bh * 4);
  p->ws.elig = take(bh);                       // uint8
  p->ws.kvis = take(bh * size_t(F + 1) * 4);   // [b][h][query frame]
  p->ws.fbound = take(bh * size_t(F + 1) * 4);
  p->ws.felig = take(bh * size_t(F + 1));      // uint8
  p->ws.qn = take(bh * size_t(p->S) * 4);      // [b][h][s]
  p->ws.qmu = take(bh * size_t(p->S) * 4);     // [b][h][s]
  p->ws.psum = take(size_t(p->nchunk) * bh * D * 4);  // [chunk][b][h][d]
  const size_t ngran = size_t(p->S) / kGranule;
  p->ws.pkmax = take(ngran * bh * 4);          // [b][h][granule], squared norms
  p->ws.pqmax = take(ngran * bh * 4);
  p->ws.kst = take(bh * size_t(D) * size_t(p->S) * 2);  // bf16 K and V, staged layouts
  p->ws.vst = take(bh * size_t(D) * size_t(p->S) * 2);
  p->ws.queue = take(kQueueWords * 4);
  const size_t nsplit_items = size_t(nsplit) * bh * p->nqb;
  p->ws.part = take(nsplit_items * 2 * part_floats(D) * 4);
  p->ws.split_cnt = take(nsplit_items * kSplitPasses * 4);
  p->ws.total = off;
  *out = p;
  return SFA_OK;
}

int check_tensor(const sfa_tensor& t) {
  if (!t.data) return SFA_ERR_INVALID;
  if (t.stride_b < 0 || t.stride_s < 0 || t.stride_h < 0) return SFA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(t.data) & 15) != 0) return SFA_ERR_UNSUPPORTED;
  if ((t.stride_b | t.stride_s | t.stride_h) & 7) return SFA_ERR_UNSUPPORTED;
  // the kernels address 64 rows of one head with 32-bit byte offsets
  if (t.stride_s > (int64_t(1) << 24)) return SFA_ERR_UNSUPPORTED;
  return SFA_OK;
}

bool ranges_overlap(const sfa_plan* p, const sfa_tensor& a, const sfa_tensor& b) {
  // conservative byte extents of two strided tensors
  auto extent = [&](const sfa_tensor& t, uintptr_t* lo, uintptr_t* hi) {
    const int64_t last = int64_t(p->g.batch - 1) * t.stride_b + int64_t(p->S - 1) * t.stride_s +
                         int64_t(p->g.heads - 1) * t.stride_h + p->g.head_dim;
    *lo = reinterpret_cast<uintptr_t>(t.data);
    *hi = *lo + uintptr_t(last) * 2;
  };
  uintptr_t alo, ahi, blo, bhi;
  extent(a, &alo, &ahi);
  extent(b, &blo, &bhi);
  return alo < bhi && blo < ahi;
}

NormParams norm_params(const sfa_plan* p, const sfa_tensor& q, const sfa_tensor& k,
                       const sfa_tensor& v, void* ws) {
  char* base = static_cast<char*>(ws);
  NormParams n;
  n.q = static_cast<const uint16_t*>(q.data);
  n.k = static_cast<const uint16_t*>(k.data);
  n.v = static_cast<const uint16_t*>(v.data);
  n.qsb = q.stride_b; n.qss = q.stride_s; n.qsh = q.stride_h;
  n.ksb = k.stride_b; n.kss = k.stride_s; n.ksh = k.stride_h;
  n.vsb = v.stride_b; n.vss = v.stride_s; n.vsh = v.stride_h;
  n.kst = reinterpret_cast<uint16_t*>(base + p->ws.kst);
  n.vst = reinterpret_cast<uint16_t*>(base + p->ws.vst);
  n.mu = reinterpret_cast<float*>(base + p->ws.mu);
  n.kmax = reinterpret_cast<float*>(base + p->ws.kmax);
  n.qmax = reinterpret_cast<float*>(base + p->ws.qmax);
  n.bound = reinterpret_cast<float*>(base + p->ws.bound);
  n.elig = reinterpret_cast<uint8_t*>(base + p->ws.elig);
  n.kvis = reinterpret_cast<float*>(base + p->ws.kvis);
  n.fbound = reinterpret_cast<float*>(base + p->ws.fbound);
  n.felig = reinterpret_cast<uint8_t*>(base + p->ws.felig);
  n.qn = reinterpret_cast<float*>(base + p->ws.qn);
  n.qmu = reinterpret_cast<float*>(base + p->ws.qmu);
  n.psum = reinterpret_cast<float*>(base + p->ws.psum);
  n.pkmax = reinterpret_cast<float*>(base + p->ws.pkmax);
  n.pqmax = reinterpret_cast<float*>(base + p->ws.pqmax);
  n.queue = reinterpret_cast<int32_t*>(base + p->ws.queue);
  n.split_cnt = reinterpret_cast<int32_t*>(base + p->ws.split_cnt);
  n.nsplit_cnt = p->nsplit * p->g.batch * p->g.heads * p->nqb * kSplitPasses;
  n.B = p->g.batch; n.H = p->g.heads; n.S = p->S; n.D = p->g.head_dim;
  n.nchunk = p->nchunk;
  n.T = p->g.tokens_per_frame; n.F = p->g.frames; n.w = p->g.window;
  n.bound_mode = p->bound_mode;
  n.scale = p->scale;
  n.bound_limit = p->g.bound_limit;
  return n;
}

// Block class for the generic ablation: 0 empty, 1 full, 2 partial. Rows
// [r0, r1) and keys [c0, c1) are the valid (unpadded) parts of the blocks; a
// block with padded keys is never full (its padding must be masked).
int generic_class(int pass, int r0, int r1, int c0, int c1, int T, int w) {
  const bool whole = c1 - c0 == kGenericBk;
  if (pass == 1) {  // reference-frame keys: every row sees them
    if (c0 >= T) return 0;
    return (c1 <= T && whole) ? 1 : 2;
  }
  const int fa = r0 / T, fb = (r1 - 1) / T, ga = c0 / T, gb = (c1 - 1) / T;
  const int a0 = fa > 1 ? fa : 1, b0 = ga > 1 ? ga : 1;
  if (a0 > fb || b0 > gb) return 0;                       // no video rows or keys
  if (a0 > gb + w || b0 > fb + w) return 0;               // frame intervals too far apart
  const bool all = fa >= 1 && ga >= 1 && whole && fb - ga <= w && gb - fa <= w;
  return all ? 1 : 2;
}

int validate_prologue(const sfa_prologue_geometry* g) {
  if (!g) return SFA_ERR_INVALID;
  if (g->batch < 1 || g->seq < 1 || g->model_dim < 1 || g->heads < 1) return SFA_ERR_INVALID;
  if (!(g->eps >= 0.0f) || !isfinite(g->eps)) return SFA_ERR_INVALID;
  if (g->head_dim != 64 && g->head_dim != 128) return SFA_ERR_UNSUPPORTED;
  if (g->model_dim % kProKStage != 0) return SFA_ERR_UNSUPPORTED;
  if ((int64_t(g->heads) * g->head_dim) % kProTile != 0) return SFA_ERR_UNSUPPORTED;
  const int64_t N = 3 * int64_t(g->heads) * g->head_dim;
  // 32-bit offsets: W' rows of one tile, tokens, feature and tile counts
  if (N * g->model_dim * 2 > (int64_t(1) << 31) - 1) return SFA_ERR_UNSUPPORTED;
  if (int64_t(g->batch) * g->seq > (int64_t(1) << 30)) return SFA_ERR_UNSUPPORTED;
  // one workgroup per 256 x 256 tile, indexed with 32-bit arithmetic
  const int64_t tiles = N / kProTile * g->batch * ((int64_t(g->seq) + kProTile - 1) / kProTile);
  if (tiles > (int64_t(1) << 31) - 1) return SFA_ERR_UNSUPPORTED;
  return SFA_OK;
}
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
}  // namespace

extern "C" {

int sfa_prologue_fold(const void* w, const void* gamma, void* w_folded, int32_t rows, int32_t cols,
                      void* stream) {
  if (!w || !gamma || !w_folded || rows < 1 || cols < 2) return SFA_ERR_INVALID;
  if (cols % 2 != 0 || !aligned16(w) || !aligned16(gamma) || !aligned16(w_folded))
    return SFA_ERR_UNSUPPORTED;
  return hip_status(sfa_launch_fold(static_cast<const uint16_t*>(w),
                                    static_cast<const uint16_t*>(gamma),
                                    static_cast<uint16_t*>(w_folded), rows, cols,
                                    static_cast<hipStream_t>(stream)));
}

int sfa_qkv_prologue(const sfa_prologue_geometry* g, sfa_tensor x, const void* w,
                     const float* cosv, const float* sinv, sfa_tensor q, sfa_tensor k, sfa_tensor v,
                     void* stream) {
  int st = validate_prologue(g);
  if (st != SFA_OK) return st;
  if (!w || !cosv || !sinv || !x.data) return SFA_ERR_INVALID;
  if (!aligned16(w) || !aligned16(cosv) || !aligned16(sinv) || !aligned16(x.data))
    return SFA_ERR_UNSUPPORTED;
  if (x.stride_b < 0 || x.stride_s < g->model_dim) return SFA_ERR_INVALID;
  if ((x.stride_b | x.stride_s) & 7) return SFA_ERR_UNSUPPORTED;
  if (x.stride_s > (int64_t(1) << 22)) return SFA_ERR_UNSUPPORTED;
  st = check_tensor(q);
  if (st == SFA_OK) st = check_tensor(k);
  if (st == SFA_OK) st = check_tensor(v);
  if (st != SFA_OK) return st;
  // the outputs may not overlap the input
  auto overlaps_x = [&](const sfa_tensor& o) {
    const uintptr_t xlo = reinterpret_cast<uintptr_t>(x.data);
    const uintptr_t xhi = xlo + uintptr_t(int64_t(g->batch - 1) * x.stride_b +
                                          int64_t(g->seq - 1) * x.stride_s + g->model_dim) * 2;
    const uintptr_t olo = reinterpret_cast<uintptr_t>(o.data);
    const uintptr_t ohi = olo + uintptr_t(int64_t(g->batch - 1) * o.stride_b +
                                          int64_t(g->seq - 1) * o.stride_s +
                                          int64_t(g->heads - 1) * o.stride_h + g->head_dim) * 2;
    return olo < xhi && xlo < ohi;
  };
  if (overlaps_x(q) || overlaps_x(k) || overlaps_x(v)) return SFA_ERR_INVALID;
  ProParams p;
  p.x = static_cast<const uint16_t*>(x.data);
  p.xsb = x.stride_b;
  p.xss = x.stride_s;
  p.w = static_cast<const uint16_t*>(w);
  p.cosv = cosv;
  p.sinv = sinv;
  const sfa_tensor* outs[3] = {&q, &k, &v};
  for (int i = 0; i < 3; ++i) {
    p.out[i] = static_cast<uint16_t*>(outs[i]->data);
    p.osb[i] = outs[i]->stride_b;
    p.oss[i] = outs[i]->stride_s;
    p.osh[i] = outs[i]->stride_h;
  }
  p.B = g->batch; p.S = g->seq; p.C = g->model_dim; p.H = g->heads; p.d = g->head_dim;
  p.ntile_f = 3 * g->heads * g->head_dim / kProTile;
  p.ntile_t = (g->seq + kProTile - 1) / kProTile;
  p.eps = g->eps;
  return hip_status(sfa_launch_prologue(p, static_cast<hipStream_t>(stream)));
}

int sfa_generic_create(const sfa_geometry* geom, sfa_generic** out) {
  if (!out) return SFA_ERR_INVALID;
  *out = nullptr;
  int st = validate_geometry(geom);
  if (st != SFA_OK) return st;
  sfa_generic* g = new (std::nothrow) sfa_generic;
  if (!g) return SFA_ERR_NOMEM;
  memset(g, 0, sizeof(*g));
  g->g = *geom;
  const int T = geom->tokens_per_frame, F = geom->frames, w = geom->window;
  const int D = geom->head_dim;
  g->scale = geom->scale == 0.0f ? 1.0f / sqrtf(float(D)) : geom->scale;
  g->S = (F + 1) * T;
  g->nqb = (g->S + kGenericBq - 1) / kGenericBq;
  g->nkb = (g->S + kGenericBk - 1) / kGenericBk;
  g->offs = static_cast<int32_t*>(malloc(sizeof(int32_t) * 2 * (g->nqb + 1)));
  // upper bound of the list length: every block of both passes
  const size_t cap = size_t(2) * g->nqb * g->nkb;
  g->lists = static_cast<int32_t*>(malloc(sizeof(int32_t) * (cap ? cap : 1)));
  if (!g->offs || !g->lists) {
    free(g->offs);
    free(g->lists);
    delete g;
    return SFA_ERR_NOMEM;
  }
  int n = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int qb = 0; qb < g->nqb; ++qb) {
      g->offs[pass * (g->nqb + 1) + qb] = n;
      const int r0 = qb * kGenericBq, r1 = std::min(g->S, r0 + kGenericBq);
      for (int kb = 0; kb < g->nkb; ++kb) {
        const int c0 = kb * kGenericBk, c1 = std::min(g->S, c0 + kGenericBk);
        const int cls = generic_class(pass, r0, r1, c0, c1, T, w);
        if (cls == 0) continue;
        g->lists[n++] = kb | (cls == 1 ? (1 << 30) : 0);
        if (cls == 1) ++g->full_blocks; else ++g->partial_blocks;
      }
    }
    g->offs[pass * (g->nqb + 1) + g->nqb] = n;
  }
  g->nlist = n;
  const int64_t bh = int64_t(geom->batch) * geom->heads;
  g->computed_pairs = (g->full_blocks + g->partial_blocks) * int64_t(kGenericBq) * kGenericBk * bh;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  g->ws_kst = take(size_t(bh) * D * size_t(g->S) * 2);
  g->ws_vst = take(size_t(bh) * D * size_t(g->S) * 2);
  g->ws_lists = take(size_t(n ? n : 1) * 4);
  g->ws_offs = take(size_t(2) * (g->nqb + 1) * 4);
  g->ws_part = take(size_t(2) * bh * size_t(g->S) * D * 4);
  g->ws_lse = take(size_t(2) * bh * size_t(g->S) * 4);
  g->ws_total = off;
  *out = g;
  return SFA_OK;
}

void sfa_generic_destroy(sfa_generic* g) {
  if (!g) return;
  free(g->lists);
  free(g->offs);
  delete g;
}

int sfa_generic_get_info(const sfa_generic* g, sfa_generic_info* out) {
  if (!g || !out) return SFA_ERR_INVALID;
  out->block_q = kGenericBq;
  out->block_k = kGenericBk;
  out->query_blocks = g->nqb;
  out->key_blocks = g->nkb;
  out->full_blocks = g->full_blocks;
  out->partial_blocks = g->partial_blocks;
  out->computed_pairs = g->computed_pairs;
  out->workspace_bytes = g->ws_total;
  return SFA_OK;
}

int sfa_generic_block_class(const sfa_generic* g, int32_t pass, int32_t qb, int32_t kb,
                            int32_t* cls) {
  if (!g || !cls || pass < 0 || pass > 1 || qb < 0 || qb >= g->nqb || kb < 0 || kb >= g->nkb)
    return SFA_ERR_INVALID;
  *cls = 0;
  for (int i = g->offs[pass * (g->nqb + 1) + qb]; i < g->offs[pass * (g->nqb + 1) + qb + 1]; ++i)
    if ((g->lists[i] & ((1 << 30) - 1)) == kb) *cls = (g->lists[i] >> 30) ? 1 : 2;
  return SFA_OK;
}

int sfa_generic_attention(const sfa_generic* g, sfa_tensor q, sfa_tensor k, sfa_tensor v,
                          sfa_tensor o, void* ws, size_t ws_bytes, void* stream) {
  if (!g || !ws) return SFA_ERR_INVALID;
  if (ws_bytes < g->ws_total) return SFA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return SFA_ERR_UNSUPPORTED;
  int st = check_tensor(q);
  if (st == SFA_OK) st = check_tensor(k);
  if (st == SFA_OK) st = check_tensor(v);
  if (st == SFA_OK) st = check_tensor(o);
  if (st != SFA_OK) return st;
  // reuse the plan-based overlap test with a plan of the same geometry
  sfa_plan tmp;
  memset(&tmp, 0, sizeof(tmp));
  tmp.g = g->g;
  tmp.S = g->S;
  if (ranges_overlap(&tmp, o, q) || ranges_overlap(&tmp, o, k) || ranges_overlap(&tmp, o, v))
    return SFA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  hipError_t e = hipMemcpyAsync(base + g->ws_lists, g->lists, size_t(g->nlist) * 4,
                                hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(base + g->ws_offs, g->offs, size_t(2) * (g->nqb + 1) * 4,
                       hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_status(e);
  NormParams n;
  memset(&n, 0, sizeof(n));
  n.k = static_cast<const uint16_t*>(k.data);
  n.ksb = k.stride_b; n.kss = k.stride_s; n.ksh = k.stride_h;
  n.v = static_cast<const uint16_t*>(v.data);
  n.vsb = v.stride_b; n.vss = v.stride_s; n.vsh = v.stride_h;
  n.kst = reinterpret_cast<uint16_t*>(base + g->ws_kst);
  n.vst = reinterpret_cast<uint16_t*>(base + g->ws_vst);
  n.B = g->g.batch; n.H = g->g.heads; n.S = g->S; n.D = g->g.head_dim;
  e = sfa_launch_stage(n, s);
  if (e != hipSuccess) return hip_status(e);
  GenericParams gp;
  gp.q = static_cast<const uint16_t*>(q.data);
  gp.k = static_cast<const uint16_t*>(k.data);
  gp.qsb = q.stride_b; gp.qss = q.stride_s; gp.qsh = q.stride_h;
  gp.ksb = k.stride_b; gp.kss = k.stride_s; gp.ksh = k.stride_h;
  gp.kst = reinterpret_cast<const uint16_t*>(base + g->ws_kst);
  gp.vst = reinterpret_cast<const uint16_t*>(base + g->ws_vst);
  gp.lists = reinterpret_cast<const int32_t*>(base + g->ws_lists);
  gp.offs = reinterpret_cast<const int32_t*>(base + g->ws_offs);
  gp.part = reinterpret_cast<float*>(base + g->ws_part);
  gp.lse = reinterpret_cast<float*>(base + g->ws_lse);
  gp.B = g->g.batch; gp.H = g->g.heads; gp.S = g->S; gp.T = g->g.tokens_per_frame;
  gp.F = g->g.frames; gp.w = g->g.window; gp.nqb = g->nqb;
  gp.items = 2 * g->g.batch * g->g.heads * g->nqb;
  gp.c = g->scale * 1.4426950408889634f;
  MergeParams m;
  m.part = gp.part;
  m.lse = gp.lse;
  m.o = static_cast<uint16_t*>(o.data);
  m.osb = o.stride_b; m.oss = o.stride_s; m.osh = o.stride_h;
  m.B = g->g.batch; m.H = g->g.heads; m.S = g->S; m.D = g->g.head_dim;
  return hip_status(sfa_launch_generic(gp, m, g->g.head_dim, s));
}

int sfa_plan_create(const sfa_geometry* geom, sfa_plan** out) {
  return create(geom, nullptr, out);
}

int sfa_plan_create_ex(const sfa_geometry* geom, const sfa_plan_options* options,
                       sfa_plan** out) {
  return create(geom, options, out);
}

void sfa_plan_destroy(sfa_plan* plan) { delete plan; }

int sfa_plan_get_info(const sfa_plan* p, sfa_plan_info* out) {
  if (!p || !out) return SFA_ERR_INVALID;
  out->block_q = p->gq * kGranule;
  out->granule = kGranule;
  out->waves_per_item = p->waves;
  out->items = p->items;
  out->active_pairs = p->active_pairs;
  out->active_flops = 4.0 * p->g.head_dim * double(p->active_pairs);
  out->io_bytes = int64_t(8) * p->g.batch * p->S * p->g.heads * p->g.head_dim;
  out->workspace_bytes = p->ws.total;
  out->bound_mode = p->bound_mode;
  out->split_frames = p->nsplit;
  out->wave_rows = 32 * p->qt;
  return SFA_OK;
}

int sfa_plan_key_ranges(const sfa_plan* p, int32_t f, int32_t ranges[4], int32_t* n) {
  if (!p || !ranges || !n) return SFA_ERR_INVALID;
  if (f < 0 || f > p->g.frames) return SFA_ERR_INVALID;
  const KeyRanges r = key_ranges(f, p->g.frames, p->g.tokens_per_frame, p->g.window);
  ranges[0] = 0;
  ranges[1] = r.r0_end;
  if (r.r1_end > r.r1_begin) {
    ranges[2] = r.r1_begin;
    ranges[3] = r.r1_end;
    *n = 2;
  } else {
    ranges[2] = ranges[3] = 0;
    *n = 1;
  }
  return SFA_OK;
}

int sfa_plan_item(const sfa_plan* p, int32_t index, int32_t item[4]) {
  if (!p || !item || index < 0 || index >= p->items) return SFA_ERR_INVALID;
  const Item it = decode_item(index, p->frame_order, p->g.batch, p->g.heads, p->nqb, p->items);
  item[0] = it.b;
  item[1] = it.h;
  item[2] = it.f;
  item[3] = it.qb;
  return SFA_OK;
}

int sfa_plan_item_keys(const sfa_plan* p, int32_t index, int32_t* half, int32_t ranges[4],
                       int32_t* n) {
  if (!p || !half || !ranges || !n || index < 0 || index >= p->items) return SFA_ERR_INVALID;
  const Item it = decode_item(index, p->frame_order, p->g.batch, p->g.heads, p->nqb, p->items);
  const int F = p->g.frames, T = p->g.tokens_per_frame, w = p->g.window;
  const KeyRanges r = it.half < 0 ? key_ranges(it.f, F, T, w) : half_key_ranges(it.f, it.half, F, T, w);
  *half = it.half;
  int m = 0;
  if (r.r0_end > 0) {
    ranges[2 * m] = 0;
    ranges[2 * m + 1] = r.r0_end;
    ++m;
  }
  if (r.r1_end > r.r1_begin) {
    ranges[2 * m] = r.r1_begin;
    ranges[2 * m + 1] = r.r1_end;
    ++m;
  }
  for (int i = 2 * m; i < 4; ++i) ranges[i] = 0;
  *n = m;
  return SFA_OK;
}

int sfa_norms(const sfa_plan* p, sfa_tensor q, sfa_tensor k, sfa_tensor v, void* ws,
              size_t ws_bytes, void* stream) {
  if (!p || !ws) return SFA_ERR_INVALID;
  if (ws_bytes < p->ws.total) return SFA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return SFA_ERR_UNSUPPORTED;
  int st = check_tensor(q);
  if (st == SFA_OK) st = check_tensor(k);
  if (st == SFA_OK) st = check_tensor(v);
  if (st != SFA_OK) return st;
  const NormParams n = norm_params(p, q, k, v, ws);
  return hip_status(sfa_launch_norms(n, static_cast<hipStream_t>(stream)));
}

int sfa_fwd(const sfa_plan* p, sfa_tensor q, sfa_tensor k, sfa_tensor v, sfa_tensor o, void* ws,
            size_t ws_bytes, void* stream) {
  if (!p || !ws) return SFA_ERR_INVALID;
  if (ws_bytes < p->ws.total) return SFA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return SFA_ERR_UNSUPPORTED;
  int st = check_tensor(q);
  if (st == SFA_OK) st = check_tensor(k);
  if (st == SFA_OK) st = check_tensor(v);
  if (st == SFA_OK) st = check_tensor(o);
  if (st != SFA_OK) return st;
  if (ranges_overlap(p, o, q) || ranges_overlap(p, o, k) || ranges_overlap(p, o, v))
    return SFA_ERR_INVALID;
  char* base = static_cast<char*>(ws);
  FwdParams f;
  f.q = static_cast<const uint16_t*>(q.data);
  f.k = static_cast<const uint16_t*>(k.data);
  f.v = static_cast<const uint16_t*>(v.data);
  f.o = static_cast<uint16_t*>(o.data);
  f.qsb = q.stride_b; f.qss = q.stride_s; f.qsh = q.stride_h;
  f.ksb = k.stride_b; f.kss = k.stride_s; f.ksh = k.stride_h;
  f.vsb = v.stride_b; f.vss = v.stride_s; f.vsh = v.stride_h;
  f.osb = o.stride_b; f.oss = o.stride_s; f.osh = o.stride_h;
  f.qn = reinterpret_cast<const float*>(base + p->ws.qn);
  f.qmu = reinterpret_cast<const float*>(base + p->ws.qmu);
  f.kvis = reinterpret_cast<const float*>(base + p->ws.kvis);
  f.felig = reinterpret_cast<const uint8_t*>(base + p->ws.felig);
  f.kst = reinterpret_cast<const uint16_t*>(base + p->ws.kst);
  f.vst = reinterpret_cast<const uint16_t*>(base + p->ws.vst);
  f.B = p->g.batch; f.H = p->g.heads; f.S = p->S; f.T = p->g.tokens_per_frame;
  f.F = p->g.frames; f.w = p->g.window;
  f.gq = p->gq; f.nqb = p->nqb; f.items = p->items;
  f.c = p->scale * 1.4426950408889634f;
  f.queue = reinterpret_cast<int32_t*>(base + p->ws.queue);
  f.part = reinterpret_cast<float*>(base + p->ws.part);
  f.split_cnt = reinterpret_cast<int32_t*>(base + p->ws.split_cnt);
  memcpy(f.frame_order, p->frame_order, sizeof(f.frame_order));
  return hip_status(
      sfa_launch_fwd(f, p->g.head_dim, p->waves, p->qt, p->stages,
                     static_cast<hipStream_t>(stream)));
}

int sfa_attention(const sfa_plan* p, sfa_tensor q, sfa_tensor k, sfa_tensor v, sfa_tensor o,
                  void* ws, size_t ws_bytes, void* stream) {
  int st = sfa_norms(p, q, k, v, ws, ws_bytes, stream);
  if (st != SFA_OK) return st;
  return sfa_fwd(p, q, k, v, o, ws, ws_bytes, stream);
}

int sfa_attention_static(const sfa_plan* p, sfa_tensor q, sfa_tensor k, sfa_tensor v,
                         sfa_tensor o, void* stream) {
  if (!p) return SFA_ERR_INVALID;
  if (p->ws.total > kStaticScratchBytes) return SFA_ERR_TOO_LARGE;
  // the stream must run on the current device: the scratch address is per device
  int dev = 0, sdev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && stream) e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
  if (e != hipSuccess) return hip_status(e);
  if (stream && sdev != dev) return SFA_ERR_INVALID;
  if (dev < 0 || dev >= kMaxDevices) return SFA_ERR_UNSUPPORTED;
  void* ws = nullptr;
  {
    // first call on this device, with the device current: the address of its copy
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      g_scratch_ptr[dev] = ptr;
    }
    ws = g_scratch_ptr[dev];
  }
  // sfa_norms writes every workspace array the attention kernel reads, the work-queue and
  // split-item counters included, so nothing left by an earlier call is used
  return sfa_attention(p, q, k, v, o, ws, kStaticScratchBytes, stream);
}

int sfa_attention_groups(const sfa_plan* p, int32_t groups, sfa_tensor q, sfa_tensor k,
                         sfa_tensor v, sfa_tensor o, void* ws, size_t ws_bytes, void* stream,
                         void* const* group_streams, int32_t nstreams) {
  if (!p || !ws || groups < 1 || nstreams < 0) return SFA_ERR_INVALID;
  if (nstreams > 0 && !group_streams) return SFA_ERR_INVALID;
  const size_t per = p->ws.total;
  if (ws_bytes / size_t(groups) < per) return SFA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return SFA_ERR_UNSUPPORTED;
  // per-group views: the same strides, data advanced by whole head groups
  auto view = [&](const sfa_tensor& t, int g) {
    sfa_tensor r = t;
    r.data = static_cast<char*>(t.data) + int64_t(g) * p->g.heads * t.stride_h * 2;
    return r;
  };
  hipStream_t main = static_cast<hipStream_t>(stream);
  const int ns = nstreams < groups ? nstreams : groups;  // streams actually used
  hipEvent_t fork = nullptr;
  hipEvent_t joins[64];
  if (ns > 64) return SFA_ERR_UNSUPPORTED;
  int st = SFA_OK;
  if (ns > 0) {
    hipError_t e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(fork, main);
    for (int i = 0; e == hipSuccess && i < ns; ++i)
      e = hipStreamWaitEvent(static_cast<hipStream_t>(group_streams[i]), fork, 0);
    if (e != hipSuccess) {
      if (fork) (void)hipEventDestroy(fork);  // already failing: report the first error
      return hip_status(e);
    }
  }
  for (int g = 0; g < groups && st == SFA_OK; ++g) {
    void* s = ns > 0 ? group_streams[g % ns] : stream;
    st = sfa_attention(p, view(q, g), view(k, g), view(v, g), view(o, g),
                       static_cast<char*>(ws) + size_t(g) * per, per, s);
  }
  if (ns > 0) {
    // join: the caller's stream waits for every group stream (also after an
    // error, so no group work is left unordered)
    int made = 0;
    hipError_t e = hipSuccess;
    for (; made < ns && e == hipSuccess; ++made) {
      e = hipEventCreateWithFlags(&joins[made], hipEventDisableTiming);
      if (e != hipSuccess) break;
      e = hipEventRecord(joins[made], static_cast<hipStream_t>(group_streams[made]));
      if (e == hipSuccess) e = hipStreamWaitEvent(main, joins[made], 0);
    }
    // destroying a recorded event is legal; its resources go once the work completes
    for (int i = 0; i <= made; ++i) {
      const hipError_t d = hipEventDestroy(i < made ? joins[i] : fork);
      if (d != hipSuccess && e == hipSuccess) e = d;
    }
    if (st == SFA_OK && e != hipSuccess) st = hip_status(e);
  }
  return st;
}

int sfa_read_head_stats(const sfa_plan* p, const void* ws, size_t ws_bytes, float* mu,
                        float* kmax, float* qmax, float* bound, uint8_t* eligible,
                        void* stream) {
  if (!p || !ws || ws_bytes < p->ws.total) return SFA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* base = static_cast<const char*>(ws);
  const size_t bh = size_t(p->g.batch) * p->g.heads;
  struct {
    void* dst;
    size_t off, bytes;
  } copies[5] = {{mu, p->ws.mu, bh * p->g.head_dim * 4},
                 {kmax, p->ws.kmax, bh * 4},
                 {qmax, p->ws.qmax, bh * 4},
                 {bound, p->ws.bound, bh * 4},
                 {eligible, p->ws.elig, bh}};
  for (auto& c : copies) {
    if (!c.dst) continue;
    hipError_t e = hipMemcpyAsync(c.dst, base + c.off, c.bytes, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(hipStreamSynchronize(s));
}

int sfa_read_frame_stats(const sfa_plan* p, const void* ws, size_t ws_bytes, float* kvis,
                         float* bound, uint8_t* eligible, void* stream) {
  if (!p || !ws || ws_bytes < p->ws.total) return SFA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* base = static_cast<const char*>(ws);
  const size_t n = size_t(p->g.batch) * p->g.heads * size_t(p->g.frames + 1);
  struct {
    void* dst;
    size_t off, bytes;
  } copies[3] = {{kvis, p->ws.kvis, n * 4}, {bound, p->ws.fbound, n * 4},
                 {eligible, p->ws.felig, n}};
  for (auto& c : copies) {
    if (!c.dst) continue;
    hipError_t e = hipMemcpyAsync(c.dst, base + c.off, c.bytes, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(hipStreamSynchronize(s));
}

int sfa_read_row_norms(const sfa_plan* p, const void* ws, size_t ws_bytes, float* qnorm,
                       float* qmu, void* stream) {
  if (!p || !ws || ws_bytes < p->ws.total) return SFA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* base = static_cast<const char*>(ws);
  const size_t bytes = size_t(p->g.batch) * p->g.heads * size_t(p->S) * 4;
  hipError_t e = hipSuccess;
  if (qnorm) e = hipMemcpyAsync(qnorm, base + p->ws.qn, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && qmu)
    e = hipMemcpyAsync(qmu, base + p->ws.qmu, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e);
}

int sfa_read_staged(const sfa_plan* p, const void* ws, size_t ws_bytes, uint16_t* k_staged,
                    uint16_t* v_staged, void* stream) {
  if (!p || !ws || ws_bytes < p->ws.total) return SFA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* base = static_cast<const char*>(ws);
  const size_t bytes = size_t(p->g.batch) * p->g.heads * size_t(p->S) * p->g.head_dim * 2;
  hipError_t e = hipSuccess;
  if (k_staged) e = hipMemcpyAsync(k_staged, base + p->ws.kst, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && v_staged)
    e = hipMemcpyAsync(v_staged, base + p->ws.vst, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e);
}

const char* sfa_status_str(int status) {
  switch (status) {
    case SFA_OK: return "ok";
    case SFA_ERR_INVALID: return "invalid argument (null pointer, bad size or workspace too small)";
    case SFA_ERR_UNSUPPORTED:
      return "unsupported (T % 16 != 0, head_dim not 64/128, misaligned pointer or stride)";
    case SFA_ERR_NOMEM: return "host allocation failed";
    case SFA_ERR_TOO_LARGE:
      return "the plan needs more workspace than sfa_attention_static's fixed 64 MiB (use "
             "sfa_attention with a caller-provided workspace)";
    case SFA_ERR_HIP:
      snprintf(g_msg, sizeof(g_msg), "HIP error %d: %s", int(g_last_hip),
               hipGetErrorString(g_last_hip));
      return g_msg;
    default: return "unknown status";
  }
}

}  // extern "C"
