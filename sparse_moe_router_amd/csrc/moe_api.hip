// C ABI of the sparse MoE layer: argument checks, workspace plan and the
// launch sequence on the caller's stream.  No allocation, no host
// synchronisation, no state kept between calls.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"
#include "moe_layer.h"

namespace moe {

namespace {

// Matrix-vector calls of up to kDecodeRows rows (bf16 experts) run the decode
// kernels, one grid row per token row, above that the small-batch kernels
// over the union of the rows' experts (measured crossover: 5 rows faster on
// the decode kernels, 6 even, 7 slower); with 4-bit experts, whose rows cost
// a quarter as much to read once per row, up to kDecodeRowsQ4.
constexpr int kDecodeRows = 5;
constexpr int kDecodeRowsQ4 = 8;

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// place `bytes` at the running offset; false on overflow
inline bool place(size_t* off, size_t* slot, uint64_t bytes) {
  *off = align256(*off);
  if (bytes > ((uint64_t)1 << 48)) return false;
  *slot = *off;
  *off += (size_t)bytes;
  return true;
}

thread_local int g_last_hip_error = 0;

moe_status_t hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Byte ranges of one call's buffers.  Every output range must be disjoint
// from every input range and from every other output range.
struct Region {
  const void* p;
  size_t n;
};
struct Regions {
  Region in[8], out[12];
  int nin = 0, nout = 0;
  void input(const void* p, size_t n) {
    if (p && n) in[nin++] = Region{p, n};
  }
  void output(const void* p, size_t n) {
    if (p && n) out[nout++] = Region{p, n};
  }
  bool disjoint() const {
    for (int i = 0; i < nout; ++i) {
      for (int j = 0; j < nin; ++j)
        if (overlap(out[i].p, out[i].n, in[j].p, in[j].n)) return false;
      for (int j = i + 1; j < nout; ++j)
        if (overlap(out[i].p, out[i].n, out[j].p, out[j].n)) return false;
    }
    return true;
  }
};

}  // namespace

bool make_plan(Plan* p, int64_t M, int H, int E, int I, int Is, int k, bool gemv) {
  memset(p, 0, sizeof(*p));
  p->M = M;
  p->H = H;
  p->E = E;
  p->I = I;
  p->Is = Is;
  p->k = k;
  p->shared = Is > 0;
  p->gemv = gemv;
  p->A = M * (int64_t)k;
  p->nchunk = (M + kChunk - 1) / kChunk;
  p->max_tiles = (p->A + kTileM - 1) / kTileM + E + (p->shared ? (M + kTileM - 1) / kTileM : 0);
  size_t off = 0;
  bool ok = true;
  if (gemv) {
    // one row: fp32 h = [k][I] routed, then [Is] shared; more rows: the
    // union lists, h = [M*k][I] per assignment, then [M][Is]
    const uint64_t A = (uint64_t)p->A;
    ok &= place(&off, &p->logits, (uint64_t)M * E * 4);
    ok &= place(&off, &p->ids, A * 4);
    ok &= place(&off, &p->w, A * 4);
    ok &= place(&off, &p->h_r, (A * I + (uint64_t)M * Is) * 4);
    if (M == 1) ok &= place(&off, &p->arrive, (uint64_t)k * kArriveStride * 4);
    if (M > 1) {
      ok &= place(&off, &p->un_count, 8);
      ok &= place(&off, &p->un_exp, (A < (uint64_t)E ? A : (uint64_t)E) * 4);
      ok &= place(&off, &p->un_off, ((A < (uint64_t)E ? A : (uint64_t)E) + 1) * 4);
      ok &= place(&off, &p->un_pair, A * 4);
      ok &= place(&off, &p->un_unit, (uint64_t)small_units(M, k, E) * 4);
    }
  } else {
    const uint64_t A = (uint64_t)p->A;
    ok &= place(&off, &p->logits, (uint64_t)M * E * 4);
    ok &= place(&off, &p->ids, A * 4);
    ok &= place(&off, &p->w, A * 4);
    ok &= place(&off, &p->cmask, (uint64_t)p->nchunk * E * 8);
    ok &= place(&off, &p->cbase, (uint64_t)p->nchunk * E * 4);
    ok &= place(&off, &p->counts, (uint64_t)E * 4);
    ok &= place(&off, &p->offsets, (uint64_t)(E + 1) * 4);
    ok &= place(&off, &p->perm, A * 4);
    ok &= place(&off, &p->inv, A * 4);
    ok &= place(&off, &p->tiles, (uint64_t)p->max_tiles * sizeof(Tile));
    ok &= place(&off, &p->ntiles, 4);
    ok &= place(&off, &p->tiles_lpt, (uint64_t)p->max_tiles * sizeof(Tile));
    ok &= place(&off, &p->h_r, A * I * 2);
    ok &= place(&off, &p->h_s, (uint64_t)M * Is * 2);
    ok &= place(&off, &p->y_r, A * H * 2);
  }
  p->total = align256(off);
  return ok;
}

}  // namespace moe

using namespace moe;

namespace {

// Shape / flag checks shared by every entry point.
moe_status_t check_desc(const moe_desc_t* d, int top_k, bool* gemv) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->M < 0) return MOE_ERR_INVALID_ARG;
  const uint32_t known = MOE_FLAG_FORCE_GEMV | MOE_FLAG_FORCE_GEMM | MOE_FLAG_TILED_WEIGHTS | MOE_FLAG_WAIT_PROBE |
                         MOE_FLAG_DECODE_TWO_LAUNCH;
  if (d->flags & ~known) return MOE_ERR_INVALID_ARG;
  if ((d->flags & MOE_FLAG_FORCE_GEMV) && (d->flags & MOE_FLAG_FORCE_GEMM)) return MOE_ERR_INVALID_ARG;
  if (d->H < 64 || d->H > 16384 || d->H % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->I < 64 || d->I > 16384 || d->I % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->I_shared < 0 || d->I_shared > 16384 || d->I_shared % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->E < 1 || d->E > kMaxE) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (top_k < 1 || top_k > d->E || top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (d->M * (int64_t)top_k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if ((d->flags & MOE_FLAG_FORCE_GEMV) && d->M > kMaxSmallM) return MOE_ERR_UNSUPPORTED_SHAPE;
  // default: one row -> decode path; up to kMaxSmallM rows averaging at most
  // kSmallRows assignments per expert -> small-batch path; else grouped
  const bool small = d->M <= kMaxSmallM && d->M * (int64_t)top_k <= (int64_t)kSmallRows * d->E;
  *gemv = (d->flags & MOE_FLAG_FORCE_GEMV) || (small && !(d->flags & MOE_FLAG_FORCE_GEMM));
  if (d->router_bias && !aligned(d->router_bias, 16)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

moe_status_t check_routing(const moe_routing_t* r) {
  if (!r) return MOE_OK;
  const void* ps[] = {r->topk_ids, r->topk_w, r->logits,    r->counts,
                      r->offsets,  r->perm,   r->tiles,     r->num_tiles, r->wait_status};
  for (const void* p : ps)
    if (p && !aligned(p, 4)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// The routing outputs' byte ranges.
void routing_regions(Regions* rg, const moe_routing_t* r, int64_t M, int E, int k, int64_t max_tiles) {
  if (!r) return;
  const size_t A = (size_t)M * k;
  rg->output(r->topk_ids, A * 4);
  rg->output(r->topk_w, A * 4);
  rg->output(r->logits, (size_t)M * E * 4);
  rg->output(r->counts, (size_t)E * 4);
  rg->output(r->offsets, (size_t)(E + 1) * 4);
  rg->output(r->perm, A * 4);
  rg->output(r->tiles, (size_t)max_tiles * sizeof(Tile));
  rg->output(r->num_tiles, 4);
  rg->output(r->wait_status, 4);
}

template <class T>
T* ws_ptr(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

SmallUnion small_union(void* ws, const Plan& p) {
  return SmallUnion{ws_ptr<int32_t>(ws, p.un_count), ws_ptr<int32_t>(ws, p.un_exp), ws_ptr<int32_t>(ws, p.un_off),
                    ws_ptr<int32_t>(ws, p.un_pair), ws_ptr<int32_t>(ws, p.un_unit)};
}

// Hands each launch the next pair of trace events (if any): the kernel is
// then launched with hipExtLaunchKernelGGL, which stamps the events with the
// kernel's own start and end.
struct Tracer {
  moe_trace_t* t;
  hipStream_t s;
  template <class F>
  hipError_t run(moe_kernel_t id, F&& fn) {
    const bool rec = t && t->count < t->capacity;
    Launch lc{s, nullptr, nullptr};
    if (rec) {
      lc.start = (hipEvent_t)t->begin[t->count];
      lc.stop = (hipEvent_t)t->end[t->count];
    }
    const hipError_t e = fn(lc);
    if (e != hipSuccess) return e;
    if (rec) {
      if (t->kernel) t->kernel[t->count] = (int32_t)id;
      t->count++;
    }
    return hipSuccess;
  }
};

// Routing on the grouped path: scores, top-k, chunk masks, scan + block map, scatter
// (the last two in one launch for calls of up to 8192 tokens).
moe_status_t run_routing_grouped(const Plan& p, const moe_desc_t* d, const void* x, const void* wr,
                                 void* ws, const moe_routing_t* r, hipStream_t s, Tracer& tr) {
  float* L = (r && r->logits) ? r->logits : ws_ptr<float>(ws, p.logits);
  int32_t* ids = (r && r->topk_ids) ? r->topk_ids : ws_ptr<int32_t>(ws, p.ids);
  float* w = (r && r->topk_w) ? r->topk_w : ws_ptr<float>(ws, p.w);
  int32_t* counts = (r && r->counts) ? r->counts : ws_ptr<int32_t>(ws, p.counts);
  int32_t* offsets = (r && r->offsets) ? r->offsets : ws_ptr<int32_t>(ws, p.offsets);
  int32_t* perm = (r && r->perm) ? r->perm : ws_ptr<int32_t>(ws, p.perm);
  Tile* tiles = (r && r->tiles) ? (Tile*)r->tiles : ws_ptr<Tile>(ws, p.tiles);
  int32_t* ntiles = (r && r->num_tiles) ? r->num_tiles : ws_ptr<int32_t>(ws, p.ntiles);
  hipError_t e;
  uint64_t* cmask = ws_ptr<uint64_t>(ws, p.cmask);
  if ((e = tr.run(MOE_K_ROUTER_SCORES, [&](const Launch& lc) {
         return launch_router_logits((const uint16_t*)x, (const uint16_t*)wr, d->router_bias, L, cmask,
                                     r ? r->wait_status : nullptr, p.M, p.H, p.E, lc);
       })) != hipSuccess)
    return hip_fail(e);
  if ((e = tr.run(MOE_K_TOPK, [&](const Launch& lc) { return launch_topk(L, ids, w, cmask, p.M, p.E, p.k, lc); })) != hipSuccess)
    return hip_fail(e);
  if (route_scan_fused(p.M)) {
    if ((e = tr.run(MOE_K_ROUTE_SCAN_SCATTER, [&](const Launch& lc) {
           return launch_route_scan_scatter(ids, cmask, counts, offsets, tiles, ntiles, ws_ptr<Tile>(ws, p.tiles_lpt),
                                            perm, ws_ptr<int32_t>(ws, p.inv), p.M, p.E, p.k, p.shared, lc);
         })) != hipSuccess)
      return hip_fail(e);
    return MOE_OK;
  }
  if ((e = tr.run(MOE_K_ROUTE_SCAN, [&](const Launch& lc) {
         return launch_route_scan(cmask, ws_ptr<int32_t>(ws, p.cbase), counts, offsets, tiles, ntiles,
                                  ws_ptr<Tile>(ws, p.tiles_lpt), p.M, p.E, p.k, p.shared, lc);
       })) != hipSuccess)
    return hip_fail(e);
  if ((e = tr.run(MOE_K_ROUTE_SCATTER, [&](const Launch& lc) {
         return launch_route_scatter(ids, ws_ptr<uint64_t>(ws, p.cmask), ws_ptr<int32_t>(ws, p.cbase), perm,
                                     ws_ptr<int32_t>(ws, p.inv), p.M, p.E, p.k, lc);
       })) != hipSuccess)
    return hip_fail(e);
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_desc_t* d, int top_k) {
  bool gemv = false;
  if (check_desc(d, top_k, &gemv) != MOE_OK) return 0;
  Plan p;
  if (!make_plan(&p, d->M, d->H, d->E, d->I, d->I_shared, top_k, gemv)) return 0;
  return p.total;
}

int64_t moe_block_map_capacity(const moe_desc_t* d, int top_k) {
  bool gemv = false;
  if (check_desc(d, top_k, &gemv) != MOE_OK) return 0;
  Plan p;
  if (!make_plan(&p, d->M, d->H, d->E, d->I, d->I_shared, top_k, false)) return 0;
  return p.max_tiles;
}

}  // extern "C"

namespace {

// Static scratch of moe_layer_forward_noalloc: the workspace of callers that
// cannot allocate.  Each device holds its own copy of this array for the
// life of the process.  On the host its name is only a stand-in: the device
// address of each device's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is passed on.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first
// call on that device); nullptr and *err set when the lookup fails.
void* scratch_for_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// The expert weights of one call: bf16 blocks, or 4-bit codes + group words.
struct Weights {
  bool q4;
  const uint16_t* ew;
  const uint16_t* sw;
  Q4Weights eq, sq;
};

moe_status_t forward_impl(const moe_desc_t* d, const void* x, const void* router_w, const Weights& wt, int top_k,
                          void* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                          const moe_routing_t* routing, moe_trace_t* trace, bool use_scratch = false) {
  bool gemv = false;
  moe_status_t st = check_desc(d, top_k, &gemv);
  if (st != MOE_OK) return st;
  if (!x || !router_w || !out) return MOE_ERR_INVALID_ARG;
  if (wt.q4) {
    if (!wt.eq.codes || !wt.eq.groups) return MOE_ERR_INVALID_ARG;
    const bool has_sh = wt.sq.codes || wt.sq.groups;
    if ((d->I_shared > 0) != has_sh || (has_sh && (!wt.sq.codes || !wt.sq.groups))) return MOE_ERR_INVALID_ARG;
    if (!aligned(wt.eq.codes, 16) || !aligned(wt.eq.groups, 16) || (has_sh && (!aligned(wt.sq.codes, 16) ||
                                                                               !aligned(wt.sq.groups, 16))))
      return MOE_ERR_MISALIGNED;
  } else {
    if (!wt.ew) return MOE_ERR_INVALID_ARG;
    if ((d->I_shared > 0) != (wt.sw != nullptr)) return MOE_ERR_INVALID_ARG;
    if (!aligned(wt.ew, 16) || (wt.sw && !aligned(wt.sw, 16))) return MOE_ERR_MISALIGNED;
  }
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(out, 16)) return MOE_ERR_MISALIGNED;
  if ((st = check_routing(routing)) != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  Plan p;
  if (!make_plan(&p, d->M, d->H, d->E, d->I, d->I_shared, top_k, gemv)) return MOE_ERR_UNSUPPORTED_SHAPE;
  p.tiled = (d->flags & MOE_FLAG_TILED_WEIGHTS) != 0;
  if (use_scratch) {
    if (p.total > kScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;  // beyond the static scratch
  } else {
    if (!workspace) return MOE_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return MOE_ERR_MISALIGNED;
    if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  {
    // outputs (out, workspace, routing buffers) disjoint from the inputs and from each other
    Regions rg;
    const size_t xbytes = (size_t)d->M * d->H * 2;
    const size_t eel = (size_t)d->E * 3 * d->I * d->H, sel = (size_t)3 * d->I_shared * d->H;
    rg.input(x, xbytes);
    rg.input(router_w, (size_t)d->E * d->H * 2);
    rg.input(d->router_bias, (size_t)d->E * 4);
    if (wt.q4) {
      rg.input(wt.eq.codes, eel / 2);
      rg.input(wt.eq.groups, eel / 16);
      rg.input(wt.sq.codes, sel / 2);
      rg.input(wt.sq.groups, sel / 16);
    } else {
      rg.input(wt.ew, eel * 2);
      rg.input(wt.sw, sel * 2);
    }
    rg.output(out, xbytes);
    rg.output(workspace, p.total);
    routing_regions(&rg, routing, d->M, d->E, top_k, p.max_tiles);
    if (!rg.disjoint()) return MOE_ERR_INVALID_ARG;
  }

  if (trace && (trace->capacity < 0 || trace->count < 0 ||
                (trace->capacity > 0 && (!trace->begin || !trace->end))))
    return MOE_ERR_INVALID_ARG;
  if (use_scratch) {  // every argument checked: the current device's static scratch is the workspace
    hipError_t err;
    workspace = scratch_for_current_device(&err);
    if (!workspace) return hip_fail(err);
  }
  hipStream_t s = stream;
  Tracer tr{trace, s};
  const uint16_t* xb = (const uint16_t*)x;
  int32_t* status = routing ? routing->wait_status : nullptr;
  hipError_t e;
  if (gemv && p.M > (wt.q4 ? kDecodeRowsQ4 : kDecodeRows)) {
    float* L = (routing && routing->logits) ? routing->logits : ws_ptr<float>(workspace, p.logits);
    int32_t* ids = (routing && routing->topk_ids) ? routing->topk_ids : ws_ptr<int32_t>(workspace, p.ids);
    float* w = (routing && routing->topk_w) ? routing->topk_w : ws_ptr<float>(workspace, p.w);
    float* h = ws_ptr<float>(workspace, p.h_r);
    const SmallUnion un = small_union(workspace, p);
    if ((e = tr.run(MOE_K_SM_ROUTER, [&](const Launch& lc) {
           return launch_small_router(xb, (const uint16_t*)router_w, d->router_bias, L, status, p, lc);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = tr.run(MOE_K_SM_TOPK, [&](const Launch& lc) { return launch_small_topk(L, ids, w, un, p, lc); })) !=
        hipSuccess)
      return hip_fail(e);
    if ((e = tr.run(MOE_K_SM_GATEUP, [&](const Launch& lc) {
           return wt.q4 ? launch_small_gateup_q4(xb, wt.eq, wt.sq, un, h, p, lc)
                        : launch_small_gateup(xb, wt.ew, wt.sw, un, h, p, lc);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = tr.run(MOE_K_SM_DOWN, [&](const Launch& lc) {
           return wt.q4 ? launch_small_down_q4(wt.eq, wt.sq, w, un, h, (uint16_t*)out, p, lc)
                        : launch_small_down(wt.ew, wt.sw, w, un, h, (uint16_t*)out, p, lc);
         })) != hipSuccess)
      return hip_fail(e);
    return MOE_OK;
  }
  if (gemv) {
    float* L = (routing && routing->logits) ? routing->logits : ws_ptr<float>(workspace, p.logits);
    int32_t* ids = (routing && routing->topk_ids) ? routing->topk_ids : ws_ptr<int32_t>(workspace, p.ids);
    float* w = (routing && routing->topk_w) ? routing->topk_w : ws_ptr<float>(workspace, p.w);
    float* h = ws_ptr<float>(workspace, p.h_r);
    if (p.M == 1 && (d->flags & MOE_FLAG_DECODE_TWO_LAUNCH) && decode_two_launch_fits(p)) {
      uint32_t* arr = ws_ptr<uint32_t>(workspace, p.arrive);
      const int probe = (d->flags & MOE_FLAG_WAIT_PROBE) ? 1 : 0;
      if ((e = tr.run(MOE_K_DEC_ROUTE, [&](const Launch& lc) {
             return wt.q4 ? launch_decode_route_q4(xb, (const uint16_t*)router_w, d->router_bias, L, wt.sq, h, arr,
                                                   status, p, lc)
                          : launch_decode_route(xb, (const uint16_t*)router_w, d->router_bias, L, wt.sw, h, arr,
                                                status, p, lc);
           })) != hipSuccess)
        return hip_fail(e);
      if ((e = tr.run(MOE_K_DEC_EXPERTS, [&](const Launch& lc) {
             return wt.q4 ? launch_decode_experts_q4(xb, wt.eq, wt.sq, L, ids, w, h, arr, status, (uint16_t*)out, p,
                                                     probe, lc)
                          : launch_decode_experts(xb, wt.ew, wt.sw, L, ids, w, h, arr, status, (uint16_t*)out, p,
                                                  probe, lc);
           })) != hipSuccess)
        return hip_fail(e);
      return MOE_OK;
    }
    if ((e = tr.run(MOE_K_DEC_ROUTER, [&](const Launch& lc) {
           return launch_decode_router(xb, (const uint16_t*)router_w, d->router_bias, L, status, p, lc);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = tr.run(MOE_K_DEC_GATEUP, [&](const Launch& lc) {
           return wt.q4 ? launch_decode_gateup_q4(xb, wt.eq, wt.sq, L, ids, w, h, p, lc)
                        : launch_decode_gateup(xb, wt.ew, wt.sw, L, ids, w, h, p, lc);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = tr.run(MOE_K_DEC_DOWN, [&](const Launch& lc) {
           return wt.q4 ? launch_decode_down_q4(wt.eq, wt.sq, ids, w, h, (uint16_t*)out, p, lc)
                        : launch_decode_down(wt.ew, wt.sw, ids, w, h, (uint16_t*)out, p, lc);
         })) != hipSuccess)
      return hip_fail(e);
    return MOE_OK;
  }
  if ((st = run_routing_grouped(p, d, x, router_w, workspace, routing, s, tr)) != MOE_OK) return st;
  const int32_t* perm = (routing && routing->perm) ? routing->perm : ws_ptr<int32_t>(workspace, p.perm);
  const float* w = (routing && routing->topk_w) ? routing->topk_w : ws_ptr<float>(workspace, p.w);
  uint16_t* h_r = ws_ptr<uint16_t>(workspace, p.h_r);
  uint16_t* h_s = ws_ptr<uint16_t>(workspace, p.h_s);
  uint16_t* y_r = ws_ptr<uint16_t>(workspace, p.y_r);
  const int32_t* inv = ws_ptr<int32_t>(workspace, p.inv);
  // with a shared expert, its tiles (the last `skip` of the block map) are left
  // out of both grouped launches: its gate/up tiles run at the start of the
  // down launch, its down GEMM carries the weighted combine in a launch of
  // its own; without one, a plain combine follows the down launch
  const int skip = p.shared ? (int)((p.M + kTileM - 1) / kTileM) : 0;
  // the block map and its count where the scan wrote them (the caller's
  // buffers when it asked for them), the gate/up launch's order of the tiles
  const Tile* tiles = (routing && routing->tiles) ? (const Tile*)routing->tiles : ws_ptr<Tile>(workspace, p.tiles);
  const int32_t* ntiles = (routing && routing->num_tiles) ? routing->num_tiles : ws_ptr<int32_t>(workspace, p.ntiles);
  const Tile* tiles_lpt = ws_ptr<Tile>(workspace, p.tiles_lpt);
  // the shared expert's gate/up tiles run at the start of the down launch (the
  // shared down + combine launch after it is the first to read their h)
  const uint16_t* x_sgu = p.shared ? xb : nullptr;
  if ((e = tr.run(MOE_K_GEMM_GATEUP, [&](const Launch& lc) {
         return wt.q4 ? launch_gemm_gateup_q4(xb, wt.eq, wt.sq, perm, tiles_lpt, ntiles, h_r, h_s, skip, p, lc)
                      : launch_gemm_gateup(xb, wt.ew, wt.sw, perm, tiles_lpt, ntiles, h_r, h_s, skip, p, lc);
       })) != hipSuccess)
    return hip_fail(e);
  if ((e = tr.run(MOE_K_GEMM_DOWN, [&](const Launch& lc) {
         return wt.q4 ? launch_gemm_down_q4(h_r, h_s, wt.eq, wt.sq, tiles, ntiles, y_r, nullptr, skip, x_sgu, p, lc)
                      : launch_gemm_down(h_r, h_s, wt.ew, wt.sw, tiles, ntiles, y_r, nullptr, skip, x_sgu, p, lc);
       })) != hipSuccess)
    return hip_fail(e);
  if (p.shared) {
    if ((e = tr.run(MOE_K_SHARED_DOWN_COMBINE, [&](const Launch& lc) {
           return wt.q4 ? launch_shared_down_combine_q4(h_s, wt.sq, y_r, w, inv, (uint16_t*)out, p, lc)
                        : launch_shared_down_combine(h_s, wt.sw, y_r, w, inv, (uint16_t*)out, p, lc);
         })) != hipSuccess)
      return hip_fail(e);
    return MOE_OK;
  }
  if ((e = tr.run(MOE_K_COMBINE, [&](const Launch& lc) {
         return launch_combine(y_r, nullptr, w, inv, (uint16_t*)out, p, lc);
       })) != hipSuccess)
    return hip_fail(e);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_layer_forward_traced(const moe_desc_t* d, const void* x, const void* router_w,
                                      const void* expert_w, const void* shared_w, int top_k,
                                      void* out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream, const moe_routing_t* routing,
                                      moe_trace_t* trace) {
  Weights wt{};
  wt.q4 = false;
  wt.ew = (const uint16_t*)expert_w;
  wt.sw = (const uint16_t*)shared_w;
  return forward_impl(d, x, router_w, wt, top_k, out, workspace, workspace_bytes, stream, routing, trace);
}

moe_status_t moe_layer_forward_q4(const moe_desc_t* d, const void* x, const void* router_w,
                                  const moe_q4_t* experts, const moe_q4_t* shared, int top_k, void* out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream,
                                  const moe_routing_t* routing, moe_trace_t* trace) {
  if (!experts) return MOE_ERR_INVALID_ARG;
  Weights wt{};
  wt.q4 = true;
  wt.eq = Q4Weights{(const uint32_t*)experts->codes, (const uint32_t*)experts->scale_bias};
  if (shared) wt.sq = Q4Weights{(const uint32_t*)shared->codes, (const uint32_t*)shared->scale_bias};
  return forward_impl(d, x, router_w, wt, top_k, out, workspace, workspace_bytes, stream, routing, trace);
}

moe_status_t moe_layer_forward(const moe_desc_t* d, const void* x, const void* router_w,
                               const void* expert_w, const void* shared_w, int top_k, void* out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream,
                               const moe_routing_t* routing) {
  return moe_layer_forward_traced(d, x, router_w, expert_w, shared_w, top_k, out, workspace,
                                  workspace_bytes, stream, routing, nullptr);
}

moe_status_t moe_layer_forward_noalloc(const moe_desc_t* d, const void* x, const void* router_w,
                                       const void* expert_w, const void* shared_w, int top_k, void* out,
                                       hipStream_t stream, const moe_routing_t* routing) {
  Weights wt{};
  wt.q4 = false;
  wt.ew = (const uint16_t*)expert_w;
  wt.sw = (const uint16_t*)shared_w;
  return forward_impl(d, x, router_w, wt, top_k, out, nullptr, 0, stream, routing, nullptr, true);
}

moe_status_t moe_route(const moe_desc_t* d, const void* x, const void* router_w, int top_k,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       const moe_routing_t* routing) {
  bool gemv = false;
  moe_status_t st = check_desc(d, top_k, &gemv);
  if (st != MOE_OK) return st;
  if (!x || !router_w || !routing) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16)) return MOE_ERR_MISALIGNED;
  if ((st = check_routing(routing)) != MOE_OK) return st;
  if (d->M == 0) return MOE_OK;
  Plan p;
  if (!make_plan(&p, d->M, d->H, d->E, d->I, d->I_shared, top_k, gemv)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return MOE_ERR_MISALIGNED;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  {
    Regions rg;
    rg.input(x, (size_t)d->M * d->H * 2);
    rg.input(router_w, (size_t)d->E * d->H * 2);
    rg.input(d->router_bias, (size_t)d->E * 4);
    rg.output(workspace, p.total);
    routing_regions(&rg, routing, d->M, d->E, top_k, p.max_tiles);
    if (!rg.disjoint()) return MOE_ERR_INVALID_ARG;
  }
  hipStream_t s = stream;
  if (gemv) {
    Plan q = p;  // selection only: no shared rows, no expert rows
    q.shared = false;
    q.Is = 0;
    q.I = 0;
    float* L = routing->logits ? routing->logits : ws_ptr<float>(workspace, p.logits);
    int32_t* ids = routing->topk_ids ? routing->topk_ids : ws_ptr<int32_t>(workspace, p.ids);
    float* w = routing->topk_w ? routing->topk_w : ws_ptr<float>(workspace, p.w);
    hipError_t e;
    if (p.M > kDecodeRows) {
      if ((e = launch_small_router((const uint16_t*)x, (const uint16_t*)router_w, d->router_bias, L,
                                   routing->wait_status, p, Launch{s, nullptr, nullptr})) != hipSuccess)
        return hip_fail(e);
      if ((e = launch_small_topk(L, ids, w, small_union(workspace, p), p, Launch{s, nullptr, nullptr})) !=
          hipSuccess)
        return hip_fail(e);
      return MOE_OK;
    }
    if ((e = launch_decode_router((const uint16_t*)x, (const uint16_t*)router_w, d->router_bias, L,
                                  routing->wait_status, q, Launch{s, nullptr, nullptr})) != hipSuccess)
      return hip_fail(e);
    if ((e = launch_decode_gateup((const uint16_t*)x, nullptr, nullptr, L, ids, w, nullptr, q,
                                  Launch{s, nullptr, nullptr})) != hipSuccess)
      return hip_fail(e);
    return MOE_OK;
  }
  Tracer none{nullptr, s};
  return run_routing_grouped(p, d, x, router_w, workspace, routing, s, none);
}

moe_status_t moe_tile_weights_q4(int64_t nblocks, int32_t H, int32_t I, const void* codes, const void* groups,
                                 void* codes_dst, void* groups_dst, hipStream_t stream) {
  if (nblocks < 0 || !codes || !groups || !codes_dst || !groups_dst) return MOE_ERR_INVALID_ARG;
  if (H < 64 || H > 16384 || H % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (I < 64 || I > 16384 || I % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!aligned(codes, 16) || !aligned(groups, 16) || !aligned(codes_dst, 16) || !aligned(groups_dst, 16))
    return MOE_ERR_MISALIGNED;
  const size_t cbytes = (size_t)nblocks * 3 * I * H / 2, gbytes = (size_t)nblocks * 3 * I * H / 16;
  Regions r;  // outputs disjoint from the inputs and from each other
  r.input(codes, cbytes);
  r.input(groups, gbytes);
  r.output(codes_dst, cbytes);
  r.output(groups_dst, gbytes);
  if (!r.disjoint()) return MOE_ERR_INVALID_ARG;
  if (nblocks == 0) return MOE_OK;
  const hipError_t e = launch_tile_weights_q4((const uint32_t*)codes, (const uint32_t*)groups, (uint32_t*)codes_dst,
                                              (uint32_t*)groups_dst, nblocks, H, I, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

moe_status_t moe_tile_weights(int64_t nblocks, int32_t H, int32_t I, const void* src, void* dst, hipStream_t stream) {
  if (nblocks < 0 || !src || !dst) return MOE_ERR_INVALID_ARG;
  if (H < 64 || H > 16384 || H % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (I < 64 || I > 16384 || I % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_MISALIGNED;
  const size_t bytes = (size_t)nblocks * 3 * I * H * 2;
  if (overlap(src, bytes, dst, bytes)) return MOE_ERR_INVALID_ARG;
  if (nblocks == 0) return MOE_OK;
  const hipError_t e = launch_tile_weights((const uint16_t*)src, (uint16_t*)dst, nblocks, H, I, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
