// C ABI of libmuon: planner, validation and launch sequence.
//
// Planner ("DMuon" 2.2 batching): matrices are bucketed by shape (m, n);
// each bucket gets the short-side orientation of "Scaling Muon for DiT" 3.1
// (transpose iff m > n), a GEMM tile size chosen from r = min(m, n), padded
// sizes r_pad / c_pad (multiples of the tile, zero filled), and is split into
// equal chunks whose Newton-Schulz scratch fits the workspace cap.  Chunks of
// a bucket run one after another and reuse one scratch region.  Buckets run
// one after another on the caller's stream, or, when all of them are too
// small to fill the device alone, concurrently on internal streams (fork /
// join through events), each stream with its own scratch region.
//
// Per chunk the refresh step enqueues:
//   prep (M update, U, ||U||^2 partials, X0 = O(U))  -> finalize (1/||U||)
//   -> SYRK G0 -> N x {POLY, PQ(+PG), PH} -> FINAL (O = Q X0, W update)
// which evaluates "Infra Optimizers" eq. (2) in the Gram space:
//   X_N = P_N ... P_1 X0,  P_k = a I + b G_{k-1} + c G_{k-1}^2,
//   G_k = P_k G_{k-1} P_k  (all P, G commute),
// with P_k = a I + P~_k, H = P G = a G + P~ G, G_k = P H = a H + P~ H and
// Q_k = P_k Q_{k-1} = a Q_{k-1} + P~_k Q_{k-1}, so every MFMA product acts on
// the non-identity part and the identity terms are added in fp32.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "kernels.h"
#include "muon.h"

using namespace muon;

namespace {

constexpr int64_t kDefaultCap = 32ll << 30;   // Newton-Schulz scratch cap (bytes)

// Tile runs per XCD for every launch of the 256-wide kernels (the hardware
// sends workgroup w to XCD w mod 8; xcd_remap_chunked gives XCD x the tiles
// [8Ck + xC, +C) of its k-th run): with runs of 32, all eight XCDs work in
// one window of 256 consecutive tiles (two to three matrices of the r x r
// products, a quarter of a final product) whose operands the shared
// last-level cache holds, while each XCD's 32 resident workgroups take
// consecutive tiles.  Found by the tuner and confirmed in same-box runs
// against the earlier rule (one contiguous range per XCD for triangular
// grids, runs of max(64, tiles per matrix / 8) for full grids).
constexpr int kXcdRun = 32;
// Concurrent buckets run on up to 4 streams: the caller's (slot 0) and up
// to 3 internal ones, so that with the default 4 hardware queues per process
// (GPU_MAX_HW_QUEUES) every stream gets a queue of its own; a fifth stream
// shares a queue with another, and its launches then wait behind that
// stream's (a kernel trace of one Qwen2.5-7B layer showed two buckets
// running one after the other that way).
constexpr int kMaxSlots = 4;
constexpr int64_t kMaxDim = 1ll << 24;        // per-dimension limit
constexpr int64_t kMaxShort = 1ll << 16;      // r = min(m, n) limit
constexpr int kRing = 4;                      // pinned descriptor staging slots
// Newton-Schulz iteration counts the paths accept.  Rounding accumulates
// with N on the 16-bit path: measured NS error 0.35-0.5e-2 at N = 6,
// 0.5-0.9e-2 at N = 12 and 0.6-2.8e-2 at N = 16 (Q's fp16 scale falls to
// 2^-13 there), so that path stops at 12, where the 2e-2 bound still holds
// with margin.  The fp32 path measured 1e-5 up to N = 16.
constexpr int kMaxSteps16 = 12;
constexpr int kMaxStepsF32 = 16;

// Operand scales (powers of two, exact) of the 16-bit Newton-Schulz path.
// Every matrix of the recursion is a polynomial in X0 X0^T, and X0 = U /
// ||U||_F has singular values sigma in [0, 1].  With f(s) = a s + b s^3 +
// c s^5 and p(g) = a + b g + c g^2, iteration k has G with eigenvalues
// g_k = f^k(sigma)^2, P~ = b G + c G^2 with b g_k + c g_k^2, H = P G with
// p(g_k) g_k, Q = P_k...P_1 with the product of p(g_j) (a^k at sigma = 0:
// padding and rank-deficient directions), and the direct form's X with
// f^k(sigma).  Entries of a symmetric matrix are bounded by its largest
// |eigenvalue|, so each scale is the largest power of two that keeps
// 1.05 x bound inside fp16's range, capped at the value that suits the
// default coefficients (for them only the Q scale depends on N: 64 up to
// N = 5, since a^5 = 484).  The bounds are taken over a grid of sigma in
// [0, 1.01] (bf16 rounding of X0 may lift sigma above 1).
constexpr float kSG = 16384.0f, kSP = 16384.0f, kSH = 8192.0f, kSQ = 64.0f, kSX = 256.0f;
constexpr double kF16Max = 65504.0;
constexpr float kMinScale = 1.0f / 16384.0f;  // below: too few fp16 bits left

struct NsScales {
  float sG = 1.0f, sP = 1.0f, sH = 1.0f, sQ = 1.0f, sX = 1.0f;
};

float pow2_fit(double bound, float cap) {
  if (!(bound > 0.0)) return cap;  // identically zero: any scale fits
  if (!std::isfinite(bound)) return 0.0f;
  const double lim = kF16Max / (1.05 * bound);
  float s = cap;
  while (s > kMinScale / 2 && (double)s > lim) s *= 0.5f;
  return s;
}

// MUON_ERR_UNSUPPORTED when the coefficients leave a bound beyond what a
// power-of-two fp16 scale can hold, or when c == 0 (the 256-tile quintic
// product folds b G into c G^2 as (b / c) G).
muon_status ns_scales(const muon_hparams& hp, NsScales* out) {
  const double a = hp.a, b = hp.b, c = hp.c;
  if (c == 0.0 || !std::isfinite(b / c) || std::fabs(b / c) > 0x1p60) return MUON_ERR_UNSUPPORTED;
  const int N = hp.ns_steps;
  double bg = 0.0, bp = 0.0, bh = 0.0, bq = 0.0, bx = 0.0;
  constexpr int kGrid = 8192;
  for (int i = 0; i <= kGrid; ++i) {
    double x = 1.01 * i / kGrid, q = 1.0;
    bx = std::max(bx, std::fabs(x));
    for (int k = 0; k < N; ++k) {
      const double g = x * x, pk = a + b * g + c * g * g;
      bg = std::max(bg, g);
      bp = std::max(bp, std::fabs(b * g + c * g * g));
      if (k < N - 1) bh = std::max(bh, std::fabs(pk * g));
      q *= pk;
      bq = std::max(bq, std::fabs(q));
      x *= pk;
      bx = std::max(bx, std::fabs(x));
    }
  }
  NsScales s;
  s.sG = pow2_fit(bg, kSG);
  s.sP = pow2_fit(bp, kSP);
  s.sH = pow2_fit(bh, kSH);
  s.sQ = pow2_fit(bq, kSQ);
  s.sX = pow2_fit(bx, kSX);
  for (float v : {s.sG, s.sP, s.sH, s.sQ, s.sX})
    if (!(v >= kMinScale)) return MUON_ERR_UNSUPPORTED;
  *out = s;
  return MUON_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Chunk {
  int first;  // index into plan order
  int count;
};

struct Bucket {
  int64_t m, n, r, c, r_pad, c_pad;
  int64_t m_pad, n_pad;  // padded natural shape (m_pad x n_pad)
  bool transposed;
  bool dma;  // 256-tile direct-to-LDS path with fp16-only r x r buffers
  bool direct;  // direct form (eq. (2) on X)
  bool fused_rr;  // Gram form with the whole r x r recursion in one launch
  bool fused_direct;  // direct form: every iteration and the update in one launch
  bool one_layout;    // rows <= cols on the 16-bit path (256-wide tiles, or the
                      // small-tile Gram form): U / X kept in the natural layout
                      // only; the products that read it across K (the final
                      // product, the 256-wide direct form's X') take it K-major
                      // through transposing LDS reads instead of a copy
  int bt;
  int group = 0, xcd = 0, waves = 0;  // 256-wide kernels' hint values (0: rule)
  int first, count;  // range in plan order
  std::vector<Chunk> chunks;
  int64_t scratch_per_mat;
  size_t chunk_scratch;  // scratch of its largest chunk
  int prep_blocks;
  int rn_row_blocks;
};

struct Slot {
  void* host = nullptr;
  hipEvent_t ev = nullptr;
  bool used = false;
};

// Host threads that enqueue the launch sequences of concurrent buckets:
// worker w runs slot w + 1 of each job (the calling thread runs slot 0).
// Created on the first concurrent call and kept until the plan is destroyed,
// so a call costs a hand-off instead of a thread start and join per slot.
struct WorkerPool {
  std::vector<std::thread> threads;
  std::mutex mu;
  std::condition_variable go, done;
  uint64_t gen = 0;  // job number; workers run each new one once
  int pending = 0;   // workers still running the current job
  bool stop = false;
  int device = 0;
  std::function<muon_status(int)> job;
  std::vector<muon_status> status;  // per slot
};

// Byte offsets of the workspace parts.  Concurrent buckets: bucket b runs on
// slot b % nslots, each slot with its own stream, scratch region and
// partial-sum region; nslots == 1: every bucket on the caller's stream.
// Streams and events are created on the first step call that needs them.
struct Layout {
  size_t off_table = 0, off_inv = 0, off_part = 0, off_colscale = 0, off_scratch = 0;
  int nslots = 1;
  std::vector<size_t> slot_scratch_off;  // bytes from off_scratch
  size_t slot_part_floats = 0;           // floats per slot from off_part
  size_t ws_bytes = 0;
};

struct TimedLaunch {
  hipEvent_t start = nullptr, stop = nullptr;
  int cls = 0;
  double flops = 0.0, bytes = 0.0;
};

}  // namespace

struct muon_plan_s {
  int64_t nmat = 0;
  muon_dtype grad_dtype = MUON_F32;
  muon_dtype ns_dtype = MUON_BF16;
  int formulation = MUON_FORM_AUTO;  // as requested; resolved per bucket
  muon_hparams hp{};
  NsScales scales;  // operand scales of the 16-bit path (all 1 on the fp32 path)
  std::vector<int64_t> rows, cols;
  std::vector<int> order;  // plan position -> caller index
  std::vector<Bucket> buckets;
  // Workspace layouts: `lay` for the caller's workspace (concurrent buckets
  // when the planner chose them), `serial` with every bucket on the caller's
  // stream (the allocation-free step's layout in the library's own scratch).
  Layout lay, serial;
  std::vector<hipStream_t> slot_streams;
  std::vector<hipEvent_t> slot_done;
  WorkerPool pool;
  hipEvent_t fork_ev = nullptr;
  // descriptor staging
  Slot ring[kRing];
  int next_slot = 0;
  bool ring_ready = false;
  std::vector<MatPtrs> host_table;
  // launch profiler (prof_active: profiling and the running call records)
  bool profiling = false;
  bool prof_active = false;
  std::vector<TimedLaunch> tpool;
  size_t tused = 0;
  double t_ms[MUON_K_COUNT] = {}, t_flops[MUON_K_COUNT] = {}, t_bytes[MUON_K_COUNT] = {};
  int64_t t_launches[MUON_K_COUNT] = {};
};

namespace {

bool finite(float x) { return std::isfinite(x); }

muon_status validate_hp(const muon_hparams& hp) {
  if (!finite(hp.momentum) || hp.momentum < 0.0f || hp.momentum > 1.0f) return MUON_ERR_INVALID_ARGUMENT;
  if (hp.nesterov != 0 && hp.nesterov != 1) return MUON_ERR_INVALID_ARGUMENT;
  if (hp.ns_steps < 1) return MUON_ERR_INVALID_ARGUMENT;
  if (hp.ns_steps > kMaxStepsF32) return MUON_ERR_UNSUPPORTED;
  if (!finite(hp.a) || !finite(hp.b) || !finite(hp.c)) return MUON_ERR_INVALID_ARGUMENT;
  if (!finite(hp.scale_coeff) || hp.scale_coeff < 0.0f) return MUON_ERR_INVALID_ARGUMENT;
  if (!finite(hp.rownorm_eps) || !(hp.rownorm_eps > 0.0f)) return MUON_ERR_INVALID_ARGUMENT;
  return MUON_OK;
}

int choose_tile(int64_t r, int64_t count, bool f32path) {
  if (r <= 64) return 64;
  if (!f32path && r > 256 && r <= 768) {
    // 256-wide tiles (the direct-to-LDS kernels) once padding r to 256 adds
    // at most 1/8 and the bucket has at least 128 lower-triangle tiles (half
    // the compute units): measured 2.3x faster than 128-wide tiles on 56
    // matrices of 512 x 3584, on par for 2 of them
    const int64_t t = (r + 255) / 256;
    if ((t * 256 - r) * 8 <= r && count * (t * (t + 1) / 2) >= 128) return 256;
  }
  if (f32path || r <= 768) {
    // small-tile path: 64-wide tiles when 128-wide ones would leave most of
    // the 256 compute units idle (under two lower-triangle tiles per CU)
    const int64_t t = (r + 127) / 128;
    return count * (t * (t + 1) / 2) < 512 ? 64 : 128;
  }
  return 256;
}

void release_ring(muon_plan_s* p) {
  for (auto& s : p->ring) {
    if (s.ev) (void)hipEventDestroy(s.ev);
    if (s.host) (void)hipHostFree(s.host);
    s.ev = nullptr;
    s.host = nullptr;
    s.used = false;
  }
  p->ring_ready = false;
}

muon_status ensure_ring(muon_plan_s* p) {
  if (p->ring_ready) return MUON_OK;
  const size_t bytes = sizeof(MatPtrs) * (size_t)p->nmat;
  for (auto& s : p->ring) {
    if (hipHostMalloc(&s.host, bytes, hipHostMallocDefault) != hipSuccess) {
      s.host = nullptr;
      release_ring(p);
      return MUON_ERR_HIP;
    }
    if (hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess) {
      s.ev = nullptr;
      release_ring(p);
      return MUON_ERR_HIP;
    }
  }
  p->ring_ready = true;
  return MUON_OK;
}

// Write the pointer table from kernel arguments (kTableChunk entries per
// launch) at dst: no staging buffer, and the stream stays on its compute
// queue (a host-to-device copy between kernels costs a copy-engine hand-off
// each way, ~15 us per call in a kernel trace of a one-matrix step).
muon_status write_table(const muon_plan_s* p, MatPtrs* dst, hipStream_t stream) {
  for (int64_t k = 0; k < p->nmat; k += kTableChunk) {
    TableChunk tc{};
    tc.count = (int)std::min<int64_t>(kTableChunk, p->nmat - k);
    for (int e = 0; e < tc.count; ++e) tc.e[e] = p->host_table[(size_t)(k + e)];
    if (launch_write_table(tc, dst + k, stream) != hipSuccess) return MUON_ERR_HIP;
  }
  return MUON_OK;
}

// Upload the per-matrix pointer table into the workspace.  Tables of up to
// kKernelTable entries (8 launches) go through write_table; larger ones
// through one host-to-device copy from a pinned ring slot that is reused only
// after its previous copy ran.
constexpr int64_t kKernelTable = 8 * kTableChunk;

muon_status upload_table(muon_plan_s* p, void* ws, hipStream_t stream) {
  if (p->nmat <= kKernelTable) return write_table(p, (MatPtrs*)((char*)ws + p->lay.off_table), stream);
  muon_status st = ensure_ring(p);
  if (st != MUON_OK) return st;
  Slot& s = p->ring[p->next_slot];
  p->next_slot = (p->next_slot + 1) % kRing;
  if (s.used && hipEventSynchronize(s.ev) != hipSuccess) return MUON_ERR_HIP;
  const size_t bytes = sizeof(MatPtrs) * (size_t)p->nmat;
  std::memcpy(s.host, p->host_table.data(), bytes);
  if (hipMemcpyAsync((char*)ws + p->lay.off_table, s.host, bytes, hipMemcpyHostToDevice, stream) !=
      hipSuccess)
    return MUON_ERR_HIP;
  if (hipEventRecord(s.ev, stream) != hipSuccess) return MUON_ERR_HIP;
  s.used = true;
  return MUON_OK;
}

// The device pointer table for this call (host_table filled), written into
// the workspace on `stream`.
muon_status table_for_call(muon_plan_s* p, void* ws, hipStream_t stream, const MatPtrs** d_table) {
  muon_status st = upload_table(p, ws, stream);
  if (st != MUON_OK) return st;
  *d_table = (const MatPtrs*)((char*)ws + p->lay.off_table);
  return MUON_OK;
}

muon_status validate_args(muon_plan_s* p, float* const* W, float* const* M, const void* const* G,
                          float lr, float wd) {
  if (!p || !W || !M || !G) return MUON_ERR_INVALID_ARGUMENT;
  if (!finite(lr) || !finite(wd)) return MUON_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < p->nmat; ++i)
    if (!W[i] || !M[i] || !G[i]) return MUON_ERR_INVALID_ARGUMENT;
  return MUON_OK;
}

muon_status validate_call(muon_plan_s* p, float* const* W, float* const* M, const void* const* G,
                          float lr, float wd, void* ws, size_t ws_bytes) {
  const muon_status st = validate_args(p, W, M, G, lr, wd);
  if (st != MUON_OK) return st;
  if (!ws || ((uintptr_t)ws & 255u) != 0) return MUON_ERR_INVALID_ARGUMENT;
  if (ws_bytes < p->lay.ws_bytes) return MUON_ERR_WORKSPACE_TOO_SMALL;
  return MUON_OK;
}

// The allocation-free step's scratch: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel or a copy (on the host it is only a
// stand-in for the symbol): it takes each device's address once, through
// hipGetSymbolAddress with that device current, and uses that.
static __device__ __align__(256) unsigned char scratch[MUON_NOALLOC_WORKSPACE_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device.
muon_status noalloc_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MUON_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MUON_ERR_HIP;
    g_scratch_dev[dev] = (char*)ptr;
  }
  *out = g_scratch_dev[dev];
  return MUON_OK;
}

// host_table is sized at plan time, so this allocates nothing.
void fill_table(muon_plan_s* p, float* const* W, float* const* M, const void* const* G,
                float* const* O) {
  for (int64_t k = 0; k < p->nmat; ++k) {
    const int i = p->order[(size_t)k];
    p->host_table[(size_t)k] = MatPtrs{W[i], M[i], G[i], O ? O[i] : nullptr};
  }
}

// Vector (16-byte) access is valid for a chunk when n is a multiple of 4 and
// every pointer of the chunk is 16-byte aligned.
int chunk_vec(const muon_plan_s* p, const Bucket& b, const Chunk& ch) {
  if (b.n % 4 != 0) return 0;
  for (int k = ch.first; k < ch.first + ch.count; ++k) {
    const MatPtrs& e = p->host_table[(size_t)k];
    const uintptr_t bits = (uintptr_t)e.W | (uintptr_t)e.M | (uintptr_t)e.G | (uintptr_t)e.O;
    if (bits & 15u) return 0;
  }
  return 1;
}

muon_status hip_ok(hipError_t e) { return e == hipSuccess ? MUON_OK : MUON_ERR_HIP; }

// Run one launch, bracketed by profiler events when profiling is enabled.
template <class F>
muon_status timed(muon_plan_s* p, hipStream_t s, int cls, double flops, double bytes, F&& launch) {
  if (!p->prof_active) return hip_ok(launch());
  if (p->tused == p->tpool.size()) {
    TimedLaunch t;
    if (hipEventCreate(&t.start) != hipSuccess) return MUON_ERR_HIP;
    if (hipEventCreate(&t.stop) != hipSuccess) {
      (void)hipEventDestroy(t.start);
      return MUON_ERR_HIP;
    }
    p->tpool.push_back(t);
  }
  TimedLaunch& t = p->tpool[p->tused++];
  t.cls = cls;
  t.flops = flops;
  t.bytes = bytes;
  if (hipEventRecord(t.start, s) != hipSuccess) return MUON_ERR_HIP;
  muon_status st = hip_ok(launch());
  if (st != MUON_OK) return st;
  return hip_ok(hipEventRecord(t.stop, s));
}

void reset_profile(muon_plan_s* p) {
  p->tused = 0;
  for (int k = 0; k < MUON_K_COUNT; ++k) {
    p->t_ms[k] = p->t_flops[k] = p->t_bytes[k] = 0.0;
    p->t_launches[k] = 0;
  }
}

void release_profile(muon_plan_s* p) {
  for (auto& t : p->tpool) {
    if (t.start) (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
  }
  p->tpool.clear();
  p->tused = 0;
}

void release_slots(muon_plan_s* p) {
  for (hipStream_t s : p->slot_streams)
    if (s) (void)hipStreamDestroy(s);
  for (hipEvent_t e : p->slot_done)
    if (e) (void)hipEventDestroy(e);
  if (p->fork_ev) (void)hipEventDestroy(p->fork_ev);
  p->slot_streams.clear();
  p->slot_done.clear();
  p->fork_ev = nullptr;
}

void stop_pool(WorkerPool& w) {
  {
    std::lock_guard<std::mutex> lock(w.mu);
    w.stop = true;
  }
  w.go.notify_all();
  for (std::thread& t : w.threads) t.join();
  w.threads.clear();
  w.stop = false;
}

void worker_main(WorkerPool* w, int slot) {
  uint64_t seen = 0;
  int cur_dev = -1;
  for (;;) {
    std::function<muon_status(int)> job;
    int dev;
    {
      std::unique_lock<std::mutex> lock(w->mu);
      w->go.wait(lock, [&] { return w->stop || w->gen != seen; });
      if (w->stop) return;
      seen = w->gen;
      job = w->job;
      dev = w->device;
    }
    // a new host thread starts on device 0: make the caller's device current
    muon_status st = MUON_OK;
    if (dev != cur_dev) {
      if (hipSetDevice(dev) == hipSuccess) cur_dev = dev;
      else st = MUON_ERR_HIP;
    }
    if (st == MUON_OK) st = job(slot);
    {
      std::lock_guard<std::mutex> lock(w->mu);
      w->status[(size_t)slot] = st;
      if (--w->pending == 0) w->done.notify_all();
    }
  }
}

// Run job(slot) for slots 0..S-1: slots 1.. on the pool's workers (started
// here on first use), slot 0 on the calling thread.  Falls back to the
// calling thread for every slot if the workers cannot be started.
muon_status run_slots(WorkerPool& w, int S, int device, const std::function<muon_status(int)>& job) {
  if ((int)w.threads.size() != S - 1) {
    stop_pool(w);
    try {
      w.status.assign((size_t)S, MUON_OK);
      for (int i = 1; i < S; ++i) w.threads.emplace_back(worker_main, &w, i);
    } catch (...) {
      stop_pool(w);
    }
  }
  if ((int)w.threads.size() != S - 1) {
    muon_status st = MUON_OK;
    for (int i = 0; i < S; ++i) {
      const muon_status v = job(i);
      if (st == MUON_OK) st = v;
    }
    return st;
  }
  {
    std::lock_guard<std::mutex> lock(w.mu);
    w.job = job;
    w.device = device;
    w.pending = S - 1;
    ++w.gen;
  }
  w.go.notify_all();
  muon_status st = job(0);
  std::unique_lock<std::mutex> lock(w.mu);
  w.done.wait(lock, [&] { return w.pending == 0; });
  for (int i = 1; i < S; ++i)
    if (st == MUON_OK) st = w.status[(size_t)i];
  w.job = nullptr;
  return st;
}

// Internal streams (default priority) of slots 1.. and their fork / join
// events (slot 0 runs on the caller's stream; its entries stay null).
muon_status ensure_slots(muon_plan_s* p) {
  if ((int)p->slot_streams.size() == p->lay.nslots) return MUON_OK;
  release_slots(p);
  if (hipEventCreateWithFlags(&p->fork_ev, hipEventDisableTiming) != hipSuccess) {
    p->fork_ev = nullptr;
    return MUON_ERR_HIP;
  }
  p->slot_streams.push_back(nullptr);
  p->slot_done.push_back(nullptr);
  for (int i = 1; i < p->lay.nslots; ++i) {
    hipStream_t s = nullptr;
    hipEvent_t e = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
      release_slots(p);
      return MUON_ERR_HIP;
    }
    p->slot_streams.push_back(s);
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      release_slots(p);
      return MUON_ERR_HIP;
    }
    p->slot_done.push_back(e);
  }
  return MUON_OK;
}

// Per-shape hints: values and duplicates checked here; whether a hint fits
// its bucket's final form is checked when the bucket is planned.
muon_status validate_hints(const muon_plan_desc* desc) {
  if (desc->num_hints < 0 || desc->num_hints > (1ll << 20)) return MUON_ERR_INVALID_ARGUMENT;
  if (desc->num_hints > 0 && !desc->hints) return MUON_ERR_INVALID_ARGUMENT;
  const bool f32path = desc->ns_dtype == MUON_F32;
  std::vector<std::pair<int64_t, int64_t>> seen;
  for (int64_t i = 0; i < desc->num_hints; ++i) {
    const muon_bucket_hint& h = desc->hints[i];
    if (h.rows < 1 || h.cols < 1) return MUON_ERR_INVALID_ARGUMENT;
    if (h.tile != 0 && h.tile != 64 && h.tile != 128 && h.tile != 256) return MUON_ERR_INVALID_ARGUMENT;
    const int f = (int)h.formulation;
    if (f != MUON_FORM_AUTO && f != MUON_FORM_GRAM && f != MUON_FORM_DIRECT)
      return MUON_ERR_INVALID_ARGUMENT;
    if (h.group < 0 || h.group > 64) return MUON_ERR_INVALID_ARGUMENT;
    if (h.xcd_chunk < -1 || h.xcd_chunk > 65536) return MUON_ERR_INVALID_ARGUMENT;
    if (h.waves != 0 && h.waves != 4 && h.waves != 8) return MUON_ERR_INVALID_ARGUMENT;
    seen.emplace_back(h.rows, h.cols);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return MUON_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < desc->num_hints; ++i) {
    const muon_bucket_hint& h = desc->hints[i];
    if (f32path && (h.tile == 256 || h.formulation == MUON_FORM_DIRECT)) return MUON_ERR_UNSUPPORTED;
  }
  return MUON_OK;
}

const muon_bucket_hint* find_hint(const muon_plan_desc* desc, int64_t m, int64_t n) {
  for (int64_t i = 0; i < desc->num_hints; ++i)
    if (desc->hints[i].rows == m && desc->hints[i].cols == n) return &desc->hints[i];
  return nullptr;
}

// Enqueue the refresh step of every bucket with workspace layout L at wsb
// and the pointer table d_table (on the device, ordered before `caller`'s
// next work), ordered after `caller`'s earlier work; `caller` waits for all
// of it.
muon_status enqueue_refresh(muon_plan_s* p, const Layout& L, char* wsb, const MatPtrs* d_table,
                            float lr, float wd, hipStream_t caller) {
  float* d_inv = (float*)(wsb + L.off_inv);
  const bool f32path = p->ns_dtype == MUON_F32;
  const int op = f32path ? OP_F32 : OP_BF16;
  const int xes = f32path ? 4 : 2;
  const int gbf16 = p->grad_dtype == MUON_BF16 ? 1 : 0;
  const muon_hparams& hp = p->hp;
  const int N = hp.ns_steps;
  const int S = L.nslots;
  muon_status st = MUON_OK;

  // fork: every slot stream waits for the table upload on the caller's stream
  if (S > 1) {
    st = ensure_slots(p);
    if (st != MUON_OK) return st;
    if (hipEventRecord(p->fork_ev, caller) != hipSuccess) return MUON_ERR_HIP;
    for (hipStream_t s : p->slot_streams)
      if (s && hipStreamWaitEvent(s, p->fork_ev, 0) != hipSuccess) return MUON_ERR_HIP;
  }
  // Enqueue the launch sequence of every bucket on slot `only_slot` (all
  // buckets when negative).
  auto run_buckets = [&](int only_slot) -> muon_status {
    muon_status st = MUON_OK;
    for (size_t bi = 0; bi < p->buckets.size(); ++bi) {
      const size_t slot = bi % (size_t)S;
      if (only_slot >= 0 && (int)slot != only_slot) continue;
      const Bucket& B = p->buckets[bi];
      const hipStream_t stream = slot > 0 ? p->slot_streams[slot] : caller;
      char* region = wsb + L.off_scratch + L.slot_scratch_off[slot];
      float* d_part = (float*)(wsb + L.off_part) + L.slot_part_floats * slot;
      const int64_t rr = B.r_pad * B.r_pad;
      const int T = (int)(B.r_pad / B.bt);
      const int ntri = T * (T + 1) / 2;
      for (const Chunk& ch : B.chunks) {
        const int nm = ch.count;
        // scratch layout for this chunk
        size_t off = 0;
        auto take = [&](size_t per_mat_bytes) {
          char* q = region + off;
          off += align256(per_mat_bytes) * (size_t)nm;
          return q;
        };
        // per-matrix strides must be uniform: use the aligned per-matrix size
        const size_t xbytes = align256((size_t)(B.r_pad * B.c_pad * xes));
        const size_t f32b = align256((size_t)(rr * 4));
        const size_t h16b = f32path ? f32b : align256((size_t)(rr * 2));
        void* Xnat = take(xbytes);  // U, m_pad x n_pad
        void* Xtr = take(xbytes);   // U^T, n_pad x m_pad
        // X0 = O(U) is r_pad x c_pad (ld c_pad); X0^T is c_pad x r_pad (ld r_pad)
        void* X = B.transposed ? Xtr : Xnat;
        void* XT = B.transposed ? Xnat : Xtr;
        float* Gf = nullptr;
        float* Qf[2] = {nullptr, nullptr};
        float* Hf = nullptr;
        if (!B.dma && !B.direct) {
          Gf = (float*)take(f32b);
          Qf[0] = (float*)take(f32b);
          Qf[1] = (float*)take(f32b);
          Hf = (float*)take(f32b);
        }
        void* Gh;
        void* Ph;
        void* Qh[2] = {nullptr, nullptr};
        void* Hh = nullptr;
        void* Xn2 = nullptr;
        void* Xt2 = nullptr;
        if (B.direct) {
          Xn2 = take(xbytes);
          Xt2 = take(xbytes);
          // the one-launch direct form keeps its r x r matrices in LDS
          Gh = B.fused_direct ? nullptr : take(h16b);
          Ph = B.fused_direct ? nullptr : take(h16b);
          if (!B.dma && !B.fused_direct) Gf = (float*)take(f32b);
        } else if (f32path) {
          Gh = Gf;
          Ph = take(f32b);
          Qh[0] = Qf[0];
          Qh[1] = Qf[1];
          Hh = Hf;
        } else {
          Gh = take(h16b);
          Ph = take(h16b);
          Qh[0] = take(h16b);
          Qh[1] = take(h16b);
          Hh = take(h16b);
        }
        const int64_t x_stride = (int64_t)(xbytes / xes);
        const int64_t rr_stride = (int64_t)(f32b / 4);
        const int64_t h_stride = (int64_t)(h16b / (f32path ? 4 : 2));
        // the epilogues index fp32 and 16-bit r x r buffers with one element
        // stride; r_pad is a multiple of 64, so both are exactly r_pad^2
        if (rr_stride != h_stride || rr_stride != rr) return MUON_ERR_HIP;
        const int vec = chunk_vec(p, B, ch);
        // W <- decay W - step_c O
        const float decay = (float)(1.0 - (double)lr * wd);
        const float step_c = (float)((double)lr * hp.scale_coeff * std::sqrt((double)B.c));
        auto gemm = [&](const GemmParams& gp, int epi) {
          if (!B.dma) return launch_gemm(gp, epi, op, B.bt, nm, stream);
          GemmParams q = gp;
          q.group = B.group;
          q.xcd_chunk = B.xcd == 0 ? kXcdRun : (B.xcd < 0 ? 0 : B.xcd);
          q.waves = (epi == EPI_SYRK || epi == EPI_FINAL) ? B.waves : 0;
          return launch_gemm_dma(q, epi, nm, stream);
        };
        // algorithmic work per matrix (true sizes; symmetric products on the
        // lower triangle): SYRK r^2 c, each r x r product r^3, final 2 r^2 c
        const double r2 = (double)B.r * B.r, r3 = r2 * B.r, cc = (double)B.c;
        const double rcf = (double)B.r * B.c;
        // algorithmic bytes per r x r element: operand reads (each operand read
        // once), the identity-term input (lower triangle, read once) and the
        // outputs (both triangles); the 256-tile path keeps only fp16 copies
        const double op_b = f32path ? 4.0 : 2.0;
        const double in_b = f32path ? 2.0 : (B.dma ? 1.0 : 2.0);
        const double out_b = f32path ? 4.0 : (B.dma ? 2.0 : 6.0);

        PrepParams pp{};
        pp.table = d_table + ch.first;
        pp.m = (int)B.m;
        pp.n = (int)B.n;
        pp.m_pad = (int)B.m_pad;
        pp.n_pad = (int)B.n_pad;
        pp.mu = hp.momentum;
        pp.nesterov = hp.nesterov;
        pp.X = Xnat;
        pp.XT = B.one_layout ? nullptr : Xtr;
        pp.x_stride = x_stride;
        pp.partials = d_part;
        pp.blocks_per_mat = B.prep_blocks;
        pp.inv_norm = d_inv + ch.first;
        const double elems = (double)B.m * B.n * nm;
        st = timed(p, stream, MUON_K_PREP, 0.0, elems * (4 + (gbf16 ? 2 : 4) + 4 + (B.one_layout ? 1 : 2) * xes), [&] {
          return launch_prep(pp, gbf16, f32path ? 1 : 0, nm, vec, stream);
        });
        if (st != MUON_OK) return st;
        if (!B.fused_direct) {  // the one-launch direct form reduces its own partials
          st = timed(p, stream, MUON_K_NORM, 0.0, 4.0 * B.prep_blocks * nm,
                     [&] { return launch_norm_finalize(pp, nm, stream); });
          if (st != MUON_OK) return st;
        }

        GemmParams g{};
        g.rr_stride = rr_stride;
        g.ldr = (int)B.r_pad;
        g.a = hp.a;
        g.b = hp.b;
        g.c = hp.c;
        g.sG = p->scales.sG;  // all 1 on the fp32 path
        g.sP = p->scales.sP;
        g.sQ = p->scales.sQ;
        g.sH = p->scales.sH;
        g.inv_norm = d_inv + ch.first;
        g.table = d_table + ch.first;
        g.Gf = Gf;
        g.Hf = Hf;
        g.Gh = Gh;
        g.Ph = Ph;
        g.Hh = Hh;
        g.products = 1;
        auto rr_setup = [&](const void* A, const void* Bop, const void* B2, int products) {
          g.A = A;
          g.B = Bop;
          g.B2 = B2;
          g.a_stride = g.b_stride = g.b2_stride = h_stride;
          g.lda = g.ldb = (int)B.r_pad;
          g.Mdim = g.Ndim = g.Kdim = (int)B.r_pad;
          g.tiles_m = g.tiles_n = T;
          g.triangular = 1;
          g.tiles_per_prod = ntri;
          g.products = products;
        };

        if (B.direct) {
          void* Xn[2] = {Xnat, Xn2};
          void* Xt[2] = {Xtr, Xt2};
          if (B.fused_direct) {
            DirectFusedParams dp{};
            dp.table = d_table + ch.first;
            dp.partials = d_part;
            dp.blocks_per_mat = B.prep_blocks;
            dp.Xn[0] = Xn[0];
            dp.Xn[1] = Xn[1];
            dp.Xt[0] = Xt[0];
            dp.Xt[1] = Xt[1];
            dp.x_stride = x_stride;
            dp.rp = (int)B.r_pad;
            dp.m = (int)B.m;
            dp.n = (int)B.n;
            dp.a = hp.a;
            dp.b = hp.b;
            dp.c = hp.c;
            dp.sX = p->scales.sX;
            dp.sG = p->scales.sG;
            dp.sP = p->scales.sP;
            dp.syrk_scale = 1.0f / (p->scales.sX * p->scales.sX);
            dp.N = N;
            dp.decay = decay;
            dp.step = step_c;
            dp.vec = vec;
            // per iteration: X^ read twice (both layouts), the a X term, X'
            // written in both layouts (the r x r matrices stay in LDS); the
            // cast reads and writes both layouts once
            st = timed(p, stream, MUON_K_XUPD, N * (r2 * cc + r3 + 2.0 * r2 * cc) * nm,
                       (N * 10.0 + 8.0) * rcf * nm, [&] { return launch_direct_fused(dp, nm, stream); });
            if (st != MUON_OK) return st;
            continue;
          }
          // X0 = U / ||U||, in place, as fp16 scaled by sX
          XcastParams xc{};
          xc.Xn = Xnat;
          xc.Xt = B.one_layout ? nullptr : Xtr;
          xc.x_stride = x_stride;
          xc.elems = B.m_pad * B.n_pad;
          xc.inv_norm = d_inv + ch.first;
          xc.sx = p->scales.sX;
          st = timed(p, stream, MUON_K_XCAST, 0.0, (B.one_layout ? 4.0 : 8.0) * (double)xc.elems * nm,
                     [&] { return launch_xcast(xc, nm, stream); });
          if (st != MUON_OK) return st;
          g.xkind = 1;
          g.syrk_scale = 1.0f / (p->scales.sX * p->scales.sX);
          g.sX = p->scales.sX;
          g.first = g.last = 0;
          const int tm = (int)(B.r_pad / B.bt), tn = (int)(B.c_pad / B.bt);
          for (int k = 0; k < N; ++k) {
            const int cur = k & 1, nx = cur ^ 1;
            void* Xk = B.transposed ? Xt[cur] : Xn[cur];    // r_pad x c_pad
            void* XTk = B.transposed ? Xn[cur] : Xt[cur];   // c_pad x r_pad
            // A = X X^T (lower tiles, mirrored)
            g.A = g.B = g.B2 = Xk;
            g.a_stride = g.b_stride = g.b2_stride = x_stride;
            g.lda = g.ldb = (int)B.c_pad;
            g.Mdim = g.Ndim = (int)B.r_pad;
            g.Kdim = (int)B.c_pad;
            g.tiles_m = g.tiles_n = T;
            g.triangular = 1;
            g.tiles_per_prod = ntri;
            g.products = 1;
            st = timed(p, stream, MUON_K_SYRK, r2 * cc * nm, (2.0 * rcf + 2.0 * r2) * nm,
                       [&] { return gemm(g, EPI_SYRK); });
            if (st != MUON_OK) return st;
            // P~ = b A + c A^2
            rr_setup(Gh, Gh, Gh, 1);
            st = timed(p, stream, MUON_K_POLY, r3 * nm, 4.0 * r2 * nm, [&] { return gemm(g, EPI_POLY); });
            if (st != MUON_OK) return st;
            // X' = a X + P~ X, written in both layouts
            GemmParams xg = g;
            xg.A = Ph;
            xg.a_stride = h_stride;
            xg.lda = (int)B.r_pad;
            xg.B = xg.B2 = B.one_layout ? Xk : XTk;  // K-major: X itself
            xg.b_stride = xg.b2_stride = x_stride;
            xg.ldb = B.one_layout ? (int)B.c_pad : (int)B.r_pad;
            xg.b_kn = B.one_layout ? 1 : 0;
            xg.Mdim = (int)B.r_pad;
            xg.Ndim = (int)B.c_pad;
            xg.Kdim = (int)B.r_pad;
            xg.tiles_m = tm;
            xg.tiles_n = tn;
            xg.triangular = 0;
            xg.tiles_per_prod = tm * tn;
            xg.products = 1;
            xg.Yn = B.transposed ? Xt[nx] : Xn[nx];
            xg.Yt = B.one_layout ? nullptr : (B.transposed ? Xn[nx] : Xt[nx]);
            xg.ldyn = (int)B.c_pad;
            xg.ldyt = (int)B.r_pad;
            xg.y_stride = x_stride;
            xg.Xid = Xk;  // the small-tile epilogue's a X term
            if (k == N - 1 && !B.transposed) {
              // X_N's tiles are W's tiles: update W from the accumulators
              // (W <- decay W - step X_N, X_N also to O_out) instead of
              // storing X_N and running the update pass
              xg.out_rows = (int)B.m;
              xg.out_cols = (int)B.n;
              xg.decay = decay;
              xg.step = step_c;
              xg.vec = vec;
              st = timed(p, stream, MUON_K_XUPD, 2.0 * r2 * cc * nm, (2.0 * r2 + 10.0 * rcf) * nm,
                         [&] { return gemm(xg, EPI_XFINAL); });
              if (st != MUON_OK) return st;
              break;
            }
            st = timed(p, stream, MUON_K_XUPD, 2.0 * r2 * cc * nm, (2.0 * r2 + (B.one_layout ? 4.0 : 6.0) * rcf) * nm,
                       [&] { return gemm(xg, EPI_XUPD); });
            if (st != MUON_OK) return st;
          }
          if (!B.transposed) continue;  // the last product updated W
          // W <- (1 - lr wd) W - lr s O^-1(X_N): the natural-layout buffer of
          // the last pair holds O^-1(X_N) in W's layout
          WupdParams wp{};
          wp.table = d_table + ch.first;
          wp.X = Xn[N & 1];
          wp.x_stride = x_stride;
          wp.m = (int)B.m;
          wp.n = (int)B.n;
          wp.n_pad = (int)B.n_pad;
          wp.inv_sx = 1.0f / p->scales.sX;
          wp.decay = decay;
          wp.step = step_c;
          st = timed(p, stream, MUON_K_WUPD, 0.0, 10.0 * (double)B.m * B.n * nm,
                     [&] { return launch_wupd(wp, nm, vec, stream); });
          if (st != MUON_OK) return st;
          continue;
        }

        // G0 = X0 X0^T / ||U||^2
        g.A = g.B = g.B2 = X;
        g.a_stride = g.b_stride = g.b2_stride = x_stride;
        g.lda = g.ldb = (int)B.c_pad;
        g.Mdim = g.Ndim = (int)B.r_pad;
        g.Kdim = (int)B.c_pad;
        g.tiles_m = g.tiles_n = T;
        g.triangular = 1;
        g.tiles_per_prod = ntri;
        g.products = 1;
        st = timed(p, stream, MUON_K_SYRK, r2 * cc * nm, (xes * rcf + r2 * out_b) * nm,
                   [&] { return gemm(g, EPI_SYRK); });
        if (st != MUON_OK) return st;

        // r_pad <= 128 on the 16-bit path: the whole recursion in one launch
        // (one workgroup per matrix) instead of up to 17 dependent launches
        const bool fused_rr = B.fused_rr;
        if (fused_rr) {
          RrFusedParams fp{};
          fp.Gf = Gf;
          fp.rr_stride = rr_stride;
          fp.r_pad = (int)B.r_pad;
          fp.Qout = Qh[(N - 1) & 1];
          fp.a = hp.a;
          fp.b = hp.b;
          fp.c = hp.c;
          fp.sG = g.sG;
          fp.sP = g.sP;
          fp.sQ = g.sQ;
          fp.sH = g.sH;
          fp.N = N;
          st = timed(p, stream, MUON_K_POLY, (4.0 * N - 3.0) * r3 * nm, 0.0,
                     [&] { return launch_rr_fused(fp, nm, stream); });
          if (st != MUON_OK) return st;
        }
        for (int k = 0; k < (fused_rr ? 0 : N); ++k) {
          const int dst = k & 1, src = dst ^ 1;
          g.first = k == 0;
          g.last = k == N - 1;
          g.Qf_src = Qf[src];
          g.Qf_dst = Qf[dst];
          g.Qh_dst = Qh[dst];
          g.Qh_src = Qh[src];
          // P~ = b G + c G^2 (and Q1 = a I + P~ on the first iteration)
          rr_setup(Gh, Gh, Gh, 1);
          st = timed(p, stream, MUON_K_POLY, r3 * nm, r2 * (op_b + in_b + out_b * (k == 0 ? 2 : 1)) * nm,
                     [&] { return gemm(g, EPI_POLY); });
          if (st != MUON_OK) return st;
          const bool need_q = k > 0;
          const bool need_h = k < N - 1;
          if (need_q || need_h) {
            // PQ: Q_k = a Q_{k-1} + P~ Q_{k-1};  PG: H = a G + P~ G
            if (need_q && need_h) {
              rr_setup(Ph, Qh[src], Gh, 2);
              g.prod_base = 0;
            } else if (need_q) {
              rr_setup(Ph, Qh[src], Qh[src], 1);
              g.prod_base = 0;
            } else {  // first iteration: Q1 came from the POLY epilogue
              rr_setup(Ph, Gh, Gh, 1);
              g.prod_base = 1;
            }
            const int np = g.products;
            st = timed(p, stream, MUON_K_PQPG, r3 * np * nm, r2 * (op_b + np * (op_b + in_b + out_b)) * nm,
                       [&] { return gemm(g, EPI_PQPG); });
            g.prod_base = 0;
            if (st != MUON_OK) return st;
          }
          if (need_h) {
            // G_k = a H + P~ H
            rr_setup(Ph, Hh, Hh, 1);
            st = timed(p, stream, MUON_K_PH, r3 * nm, r2 * (2 * op_b + in_b + out_b) * nm,
                       [&] { return gemm(g, EPI_PH); });
            if (st != MUON_OK) return st;
          }
        }

        // O = Q X0 / ||U||;  W <- (1 - lr wd) W - lr s O   (with O^-1 orientation)
        const void* Qfinal = f32path ? (const void*)Qf[(N - 1) & 1] : (const void*)Qh[(N - 1) & 1];
        GemmParams fg = g;
        fg.Kdim = (int)B.r_pad;
        fg.triangular = 0;
        fg.products = 1;
        fg.vec = vec;
        fg.out_rows = (int)B.m;
        fg.out_cols = (int)B.n;
        fg.decay = decay;
        fg.step = step_c;
        if (!B.transposed) {  // O (r x c) = Q (r x r) * (X0^T)^T
          fg.A = Qfinal;
          fg.a_stride = h_stride;
          fg.lda = (int)B.r_pad;
          fg.B = fg.B2 = B.one_layout ? X : XT;  // K-major: X0 itself
          fg.b_stride = fg.b2_stride = x_stride;
          fg.ldb = B.one_layout ? (int)B.c_pad : (int)B.r_pad;
          fg.b_kn = B.one_layout ? 1 : 0;
          fg.Mdim = (int)B.r_pad;
          fg.Ndim = (int)B.c_pad;
        } else {  // O^T (c x r) = X0^T (c x r) * Q
          fg.A = XT;
          fg.a_stride = x_stride;
          fg.lda = (int)B.r_pad;
          fg.B = fg.B2 = Qfinal;
          fg.b_stride = fg.b2_stride = h_stride;
          fg.ldb = (int)B.r_pad;
          fg.Mdim = (int)B.c_pad;
          fg.Ndim = (int)B.r_pad;
        }
        fg.tiles_m = fg.Mdim / B.bt;
        fg.tiles_n = fg.Ndim / B.bt;
        fg.tiles_per_prod = fg.tiles_m * fg.tiles_n;
        st = timed(p, stream, MUON_K_FINAL, 2.0 * r2 * cc * nm, (xes * rcf + op_b * r2 + 8.0 * rcf) * nm,
                   [&] { return gemm(fg, EPI_FINAL); });
        if (st != MUON_OK) return st;
      }
    }
    return MUON_OK;
  };
  int dev = -1;
  if (S > 1 && !p->prof_active && hipGetDevice(&dev) == hipSuccess) {
    // Each slot's launch sequence is enqueued from its own host thread, so
    // that every slot's first kernels reach the GPU at once instead of after
    // the whole sequence of the slots before it (~13 us of host time per
    // launch; one Qwen2.5-7B layer: 8.3 -> 7.9 ms per step).  The threads
    // only read the plan and launch on distinct streams.
    st = run_slots(p->pool, S, dev, run_buckets);
  } else {
    st = run_buckets(-1);
  }
  // join: the caller's stream waits for every slot (also after a failed
  // launch, so that no work of this call is left unordered)
  if (S > 1) {
    for (int i = 1; i < S; ++i) {
      if (hipEventRecord(p->slot_done[(size_t)i], p->slot_streams[(size_t)i]) != hipSuccess ||
          hipStreamWaitEvent(caller, p->slot_done[(size_t)i], 0) != hipSuccess)
        st = MUON_ERR_HIP;
    }
  }
  return st;
}

}  // namespace

extern "C" {

muon_status muon_default_hparams(muon_hparams* hp) {
  if (!hp) return MUON_ERR_INVALID_ARGUMENT;
  hp->momentum = 0.95f;
  hp->nesterov = 1;
  hp->ns_steps = 5;
  hp->a = 3.4445f;
  hp->b = -4.7750f;
  hp->c = 2.0315f;
  hp->scale_coeff = 0.2f;
  hp->rownorm_eps = 1e-8f;
  return MUON_OK;
}

const char* muon_status_string(muon_status s) {
  switch (s) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARGUMENT: return "MUON_ERR_INVALID_ARGUMENT";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_WORKSPACE_TOO_SMALL: return "MUON_ERR_WORKSPACE_TOO_SMALL";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
  }
  return "MUON_UNKNOWN_STATUS";
}

muon_status muon_plan(const muon_plan_desc* desc, muon_plan_t* plan, size_t* workspace_bytes) {
  if (!desc || !plan) return MUON_ERR_INVALID_ARGUMENT;
  *plan = nullptr;
  if (desc->num_matrices < 1 || !desc->rows || !desc->cols) return MUON_ERR_INVALID_ARGUMENT;
  if (desc->num_matrices > (1ll << 24)) return MUON_ERR_UNSUPPORTED;
  if (desc->grad_dtype != MUON_F32 && desc->grad_dtype != MUON_BF16) return MUON_ERR_INVALID_ARGUMENT;
  if (desc->ns_dtype != MUON_F32 && desc->ns_dtype != MUON_BF16) return MUON_ERR_INVALID_ARGUMENT;
  if (desc->max_workspace_bytes < 0) return MUON_ERR_INVALID_ARGUMENT;
  const int form = (int)desc->formulation;
  if (form != MUON_FORM_AUTO && form != MUON_FORM_GRAM && form != MUON_FORM_DIRECT)
    return MUON_ERR_INVALID_ARGUMENT;
  if (form == MUON_FORM_DIRECT && desc->ns_dtype == MUON_F32) return MUON_ERR_UNSUPPORTED;
  muon_status st = validate_hp(desc->hp);
  if (st != MUON_OK) return st;
  NsScales scales;
  if (desc->ns_dtype == MUON_BF16) {
    if (desc->hp.ns_steps > kMaxSteps16) return MUON_ERR_UNSUPPORTED;
    st = ns_scales(desc->hp, &scales);
    if (st != MUON_OK) return st;
  }
  for (int64_t i = 0; i < desc->num_matrices; ++i) {
    const int64_t m = desc->rows[i], n = desc->cols[i];
    if (m < 1 || n < 1) return MUON_ERR_INVALID_ARGUMENT;
    if (m > kMaxDim || n > kMaxDim || std::min(m, n) > kMaxShort) return MUON_ERR_UNSUPPORTED;
  }
  st = validate_hints(desc);
  if (st != MUON_OK) return st;
  muon_plan_s* p = nullptr;
  try {
    p = new muon_plan_s();
    p->nmat = desc->num_matrices;
    p->grad_dtype = desc->grad_dtype;
    p->ns_dtype = desc->ns_dtype;
    p->hp = desc->hp;
    p->scales = scales;
    p->rows.assign(desc->rows, desc->rows + desc->num_matrices);
    p->cols.assign(desc->cols, desc->cols + desc->num_matrices);
    const bool f32path = desc->ns_dtype == MUON_F32;
    p->formulation = form;
    const int64_t cap = desc->max_workspace_bytes > 0 ? desc->max_workspace_bytes : kDefaultCap;

    // buckets in order of first appearance
    std::vector<std::vector<int>> members;
    for (int64_t i = 0; i < p->nmat; ++i) {
      size_t b = 0;
      for (; b < p->buckets.size(); ++b)
        if (p->buckets[b].m == p->rows[i] && p->buckets[b].n == p->cols[i]) break;
      if (b == p->buckets.size()) {
        Bucket nb{};
        nb.m = p->rows[i];
        nb.n = p->cols[i];
        p->buckets.push_back(nb);
        members.emplace_back();
      }
      members[b].push_back((int)i);
    }
    size_t part_floats = 0, colscale_floats = 0, max_scratch = 0;
    for (size_t b = 0; b < p->buckets.size(); ++b) {
      Bucket& B = p->buckets[b];
      B.transposed = B.m > B.n;
      B.r = std::min(B.m, B.n);
      B.c = std::max(B.m, B.n);
      // AUTO: the direct form for near-square matrices (c <= 1.125 r) on the
      // 16-bit path, the Gram form otherwise (3 r^2 c + 17 r^3 against
      // 15 r^2 c + 5 r^3 flops for c > r).  Near-square inputs have singular
      // values close to zero, which the Gram form's squared spectrum resolves
      // badly in fp16: measured over r = 40..1000 (worst of two seeds, both
      // orientations) the Gram form's NS error is 1.1e-2..3.2e-2 on squares
      // and 0.8e-2 at worst from c > 1.125 r on, the direct form's 0.25e-2..
      // 0.64e-2 everywhere; on squares the two cost the same 20 r^3 flops
      // and the direct form measured 2-10 % faster (3.6x on 64 x 512^2).
      const bool near_square = 8 * B.c <= 9 * B.r;
      B.direct = p->formulation == MUON_FORM_DIRECT ||
                 (p->formulation == MUON_FORM_AUTO && !f32path && near_square);
      const muon_bucket_hint* hint = find_hint(desc, B.m, B.n);
      if (hint && hint->formulation != MUON_FORM_AUTO) B.direct = hint->formulation == MUON_FORM_DIRECT;
      if (!f32path && !B.direct && near_square) {
        // a Gram form forced onto a near-square bucket on the 16-bit path
        // would miss the accuracy the path promises (see above)
        delete p;
        return MUON_ERR_UNSUPPORTED;
      }
      // the direct form takes the same tile rule: 64- or 128-wide tiles (the
      // small-tile kernel) for small r, 256-wide ones above
      B.bt = choose_tile(B.r, (int64_t)members[b].size(), f32path);
      if (hint && hint->tile != 0) B.bt = hint->tile;
      if (hint) {
        B.group = hint->group;
        B.xcd = hint->xcd_chunk;
        B.waves = hint->waves;
        // the knobs of the 256-wide kernels need those kernels
        if ((B.group || B.xcd || B.waves) && (f32path || B.bt != 256)) {
          delete p;
          return MUON_ERR_UNSUPPORTED;
        }
      }
      B.r_pad = round_up(B.r, B.bt);
      B.c_pad = round_up(B.c, B.bt);
      B.first = (int)p->order.size();
      B.count = (int)members[b].size();
      for (int i : members[b]) p->order.push_back(i);
      const int64_t xes = f32path ? 4 : 2;
      const int64_t rr = B.r_pad * B.r_pad;
      B.dma = !f32path && B.bt == 256;
      B.fused_rr = !f32path && !B.dma && !B.direct && B.r_pad <= 128;
      // padded squares of 128 or 256 on the small-tile 16-bit path: the
      // direct form's 3 N products and the update in one launch
      B.fused_direct = !f32path && !B.dma && B.direct && !B.transposed && B.r_pad == B.c_pad &&
                       (B.r_pad == 128 || B.r_pad == 256);
      // rows <= cols on the 16-bit path: the products that would read X0^T
      // (the final product, the 256-wide direct form's X') read X0 across K
      // instead; the small-tile direct form keeps both layouts
      B.one_layout = !f32path && !B.transposed && (B.dma || !B.direct);
      // r x r buffers: fp32 path: G, Q x2, H, P~ in fp32; bf16 path: fp32
      // master copies G, Q x2, H plus fp16 operand copies G, P~, Q x2, H;
      // the 256-tile path keeps only the fp16 copies
      const int64_t rr_bytes =
          f32path ? 5 * (int64_t)align256((size_t)(rr * 4))
                  : (B.dma ? 0 : 4 * (int64_t)align256((size_t)(rr * 4))) +
                        5 * (int64_t)align256((size_t)(rr * 2));
      const int64_t xb = (int64_t)align256((size_t)(B.r_pad * B.c_pad * xes));
      // direct form: X and X^T twice (double buffered) plus A and P~ in fp16
      // (and A in fp32 for the small-tile kernel's quintic epilogue)
      B.scratch_per_mat = B.fused_direct ? 4 * xb
                        : B.direct ? 4 * xb + 2 * (int64_t)align256((size_t)(rr * 2)) +
                                         (B.dma ? 0 : (int64_t)align256((size_t)(rr * 4)))
                                   : 2 * xb + rr_bytes;
      int64_t per_chunk = std::max<int64_t>(1, cap / B.scratch_per_mat);
      per_chunk = std::min<int64_t>(per_chunk, B.count);
      const int64_t nchunks = (B.count + per_chunk - 1) / per_chunk;
      const int64_t even = (B.count + nchunks - 1) / nchunks;
      for (int64_t f = 0; f < B.count; f += even)
        B.chunks.push_back(Chunk{B.first + (int)f, (int)std::min<int64_t>(even, B.count - f)});
      B.m_pad = B.transposed ? B.c_pad : B.r_pad;
      B.n_pad = B.transposed ? B.r_pad : B.c_pad;
      B.prep_blocks = prep_blocks_per_mat((int)B.m_pad, (int)B.n_pad, B.one_layout);
      B.rn_row_blocks = rownorm_row_blocks((int)B.m, (int)B.n);
      B.chunk_scratch = (size_t)(even * B.scratch_per_mat);
      max_scratch = std::max(max_scratch, B.chunk_scratch);
      part_floats = std::max(part_floats, (size_t)even * (size_t)B.prep_blocks);
      if (B.transposed) {
        // RowNorm runs on whole buckets (no NS scratch needed)
        part_floats = std::max(part_floats, (size_t)B.count * B.rn_row_blocks * (size_t)B.n);
        colscale_floats = std::max(colscale_floats, (size_t)B.count * (size_t)B.n);
      }
    }
    // Buckets too small to fill the device on their own (one launch chunk,
    // every r x r product under two waves of workgroups for the 256 compute
    // units: a compute unit holds one 256-wide tile's workgroup, two of the
    // 128-wide kernel and four of the 64-wide one) run concurrently on up to
    // kMaxSlots streams when their scratch regions fit the cap together;
    // otherwise all run one after another.
    const int nb = (int)p->buckets.size();
    bool small = nb > 1;
    for (const Bucket& B : p->buckets) {
      const int64_t T = B.r_pad / B.bt;
      const int64_t per_cu = B.bt == 256 ? 1 : (B.bt == 128 ? 2 : 4);
      if (B.chunks.size() != 1 || (int64_t)B.count * (T * (T + 1) / 2) >= 512 * per_cu) small = false;
    }
    int S = small ? std::min(nb, kMaxSlots) : 1;
    std::vector<size_t> slot_bytes((size_t)S, 0);
    for (int b = 0; b < nb; ++b)
      slot_bytes[(size_t)(b % S)] = std::max(slot_bytes[(size_t)(b % S)],
                                             align256(p->buckets[(size_t)b].chunk_scratch));
    size_t total = 0;
    for (size_t v : slot_bytes) total += v;
    if (S > 1 && total > (size_t)cap) {
      S = 1;
      slot_bytes.assign(1, max_scratch);
      total = max_scratch;
    }
    auto layout = [&](const std::vector<size_t>& bytes) {
      Layout L;
      const int nsl = (int)bytes.size();
      L.nslots = nsl;
      L.slot_scratch_off.assign((size_t)nsl, 0);
      size_t tot = 0;
      for (size_t i = 0; i < bytes.size(); ++i) {
        L.slot_scratch_off[i] = tot;
        tot += bytes[i];
      }
      L.slot_part_floats = align256(sizeof(float) * std::max<size_t>(part_floats, 1)) / sizeof(float);
      L.off_table = 0;
      L.off_inv = align256(sizeof(MatPtrs) * (size_t)p->nmat);
      L.off_part = L.off_inv + align256(sizeof(float) * (size_t)p->nmat);
      L.off_colscale = L.off_part + sizeof(float) * L.slot_part_floats * (size_t)nsl;
      L.off_scratch = L.off_colscale + align256(sizeof(float) * std::max<size_t>(colscale_floats, 1));
      L.ws_bytes = L.off_scratch + tot;
      return L;
    };
    p->lay = layout(slot_bytes);
    p->serial = layout(std::vector<size_t>(1, max_scratch));
    p->host_table.resize((size_t)p->nmat);
  } catch (const std::bad_alloc&) {
    delete p;
    return MUON_ERR_INVALID_ARGUMENT;
  }
  *plan = p;
  if (workspace_bytes) *workspace_bytes = p->lay.ws_bytes;
  return MUON_OK;
}

muon_status muon_plan_destroy(muon_plan_t plan) {
  if (!plan) return MUON_OK;
  stop_pool(plan->pool);
  release_ring(plan);
  release_profile(plan);
  release_slots(plan);
  delete plan;
  return MUON_OK;
}

muon_status muon_plan_workspace_size(muon_plan_t plan, size_t* workspace_bytes) {
  if (!plan || !workspace_bytes) return MUON_ERR_INVALID_ARGUMENT;
  *workspace_bytes = plan->lay.ws_bytes;
  return MUON_OK;
}

muon_status muon_plan_info(muon_plan_t plan, int64_t* num_buckets, int64_t* num_chunks) {
  if (!plan) return MUON_ERR_INVALID_ARGUMENT;
  int64_t nc = 0;
  for (const auto& b : plan->buckets) nc += (int64_t)b.chunks.size();
  if (num_buckets) *num_buckets = (int64_t)plan->buckets.size();
  if (num_chunks) *num_chunks = nc;
  return MUON_OK;
}

muon_status muon_plan_bucket_info(muon_plan_t plan, int64_t index, muon_bucket_info* info) {
  if (!plan || !info || index < 0 || index >= (int64_t)plan->buckets.size())
    return MUON_ERR_INVALID_ARGUMENT;
  const Bucket& B = plan->buckets[(size_t)index];
  info->rows = B.m;
  info->cols = B.n;
  info->count = B.count;
  info->chunks = (int64_t)B.chunks.size();
  info->tile = B.bt;
  info->formulation = B.direct ? MUON_FORM_DIRECT : MUON_FORM_GRAM;
  info->transposed = B.transposed ? 1 : 0;
  info->fused_recursion = (B.fused_rr || B.fused_direct) ? 1 : 0;
  const NsScales& sc = plan->scales;
  const float scales[5] = {sc.sG, sc.sP, sc.sH, sc.sQ, sc.sX};
  std::memcpy(info->operand_scales, scales, sizeof scales);
  info->group = B.group;
  info->xcd_chunk = B.xcd;
  info->waves = B.waves;
  return MUON_OK;
}

muon_status muon_step_batched(muon_plan_t p, float* const* W, float* const* M, const void* const* G,
                              float lr, float wd, void* ws, size_t ws_bytes, hipStream_t stream,
                              float* const* O_out) {
  muon_status st = validate_call(p, W, M, G, lr, wd, ws, ws_bytes);
  if (st != MUON_OK) return st;
  try {
    fill_table(p, W, M, G, O_out);
  } catch (const std::bad_alloc&) {
    return MUON_ERR_INVALID_ARGUMENT;
  }
  const MatPtrs* d_table = nullptr;
  st = table_for_call(p, ws, stream, &d_table);
  if (st != MUON_OK) return st;
  p->prof_active = p->profiling;
  return enqueue_refresh(p, p->lay, (char*)ws, d_table, lr, wd, stream);
}

muon_status muon_step_batched_noalloc(muon_plan_t p, float* const* W, float* const* M,
                                      const void* const* G, float lr, float wd, hipStream_t stream,
                                      float* const* O_out) {
  muon_status st = validate_args(p, W, M, G, lr, wd);
  if (st != MUON_OK) return st;
  if (p->serial.ws_bytes > (size_t)MUON_NOALLOC_WORKSPACE_BYTES) return MUON_ERR_WORKSPACE_TOO_SMALL;
  char* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != MUON_OK) return st;
  fill_table(p, W, M, G, O_out);
  // the pointer table reaches the scratch as kernel arguments: no staging
  // buffer, and ordered on the stream like the rest of the step
  st = write_table(p, (MatPtrs*)(ws + p->serial.off_table), stream);
  if (st != MUON_OK) return st;
  p->prof_active = false;
  return enqueue_refresh(p, p->serial, ws, (const MatPtrs*)(ws + p->serial.off_table), lr, wd, stream);
}

muon_status rownorm_step(muon_plan_t p, float* const* W, float* const* M, const void* const* G,
                         float lr, float wd, void* ws, size_t ws_bytes, hipStream_t stream,
                         float* const* R_out) {
  muon_status st = validate_call(p, W, M, G, lr, wd, ws, ws_bytes);
  if (st != MUON_OK) return st;
  try {
    fill_table(p, W, M, G, R_out);
  } catch (const std::bad_alloc&) {
    return MUON_ERR_INVALID_ARGUMENT;
  }
  const MatPtrs* d_table = nullptr;
  st = table_for_call(p, ws, stream, &d_table);
  if (st != MUON_OK) return st;
  p->prof_active = p->profiling;
  char* wsb = (char*)ws;
  const int gbf16 = p->grad_dtype == MUON_BF16 ? 1 : 0;
  for (const Bucket& B : p->buckets) {
    RowNormParams rp{};
    rp.table = d_table + B.first;
    rp.m = (int)B.m;
    rp.n = (int)B.n;
    rp.mu = p->hp.momentum;
    rp.nesterov = p->hp.nesterov;
    rp.eps = p->hp.rownorm_eps;
    rp.decay = (float)(1.0 - (double)lr * wd);
    rp.step = (float)((double)lr * p->hp.scale_coeff * std::sqrt((double)B.c));
    rp.partials = (float*)(wsb + p->lay.off_part);
    rp.colscale = (float*)(wsb + p->lay.off_colscale);
    rp.row_blocks = B.rn_row_blocks;
    const int vec = chunk_vec(p, B, Chunk{B.first, B.count});
    const double elems = (double)B.m * B.n * B.count;
    const double gb = gbf16 ? 2.0 : 4.0;
    const int nm = B.count;
    if (!B.transposed) {
      // read M, G, W; write M, W
      st = timed(p, stream, MUON_K_ROWNORM, 0.0, elems * (4 + gb + 4 + 4 + 4), [&] {
        return launch_rownorm(rp, gbf16, nm, vec, RN_PHASE_ROWS, stream);
      });
      if (st != MUON_OK) return st;
      continue;
    }
    st = timed(p, stream, MUON_K_COLSUM, 0.0, elems * (4 + gb + 4), [&] {
      return launch_rownorm(rp, gbf16, nm, vec, RN_PHASE_COLSUM, stream);
    });
    if (st != MUON_OK) return st;
    st = timed(p, stream, MUON_K_COLFINAL, 0.0, 4.0 * (B.rn_row_blocks + 1) * B.n * nm, [&] {
      return launch_rownorm(rp, gbf16, nm, vec, RN_PHASE_COLFINAL, stream);
    });
    if (st != MUON_OK) return st;
    st = timed(p, stream, MUON_K_COLAPPLY, 0.0, elems * (4 + gb + 4 + 4), [&] {
      return launch_rownorm(rp, gbf16, nm, vec, RN_PHASE_COLAPPLY, stream);
    });
    if (st != MUON_OK) return st;
  }
  return MUON_OK;
}

muon_status muon_plan_set_profiling(muon_plan_t plan, int enable) {
  if (!plan || (enable != 0 && enable != 1)) return MUON_ERR_INVALID_ARGUMENT;
  plan->profiling = enable == 1;
  reset_profile(plan);
  return MUON_OK;
}

muon_status muon_plan_kernel_times(muon_plan_t plan, double* total_ms, int64_t* launches,
                                   double* flops, double* bytes) {
  if (!plan) return MUON_ERR_INVALID_ARGUMENT;
  for (size_t i = 0; i < plan->tused; ++i) {
    TimedLaunch& t = plan->tpool[i];
    float ms = 0.0f;
    if (hipEventSynchronize(t.stop) != hipSuccess) return MUON_ERR_HIP;
    if (hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) return MUON_ERR_HIP;
    plan->t_ms[t.cls] += ms;
    plan->t_flops[t.cls] += t.flops;
    plan->t_bytes[t.cls] += t.bytes;
    plan->t_launches[t.cls] += 1;
  }
  plan->tused = 0;
  for (int k = 0; k < MUON_K_COUNT; ++k) {
    if (total_ms) total_ms[k] = plan->t_ms[k];
    if (launches) launches[k] = plan->t_launches[k];
    if (flops) flops[k] = plan->t_flops[k];
    if (bytes) bytes[k] = plan->t_bytes[k];
  }
  return MUON_OK;
}

}  // extern "C"
