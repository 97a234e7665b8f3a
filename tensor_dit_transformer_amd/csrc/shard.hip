// Host layer of the C ABI declared in include/tp_shard.h: argument
// validation, the rank's weight-slice upload, and kernel launches on the
// caller's stream.  Validation comes first everywhere and nothing is
// enqueued on error ("raise instead of silently doing something else",
// Diffusers TP page, §Limitações; "check before loading or splitting any
// weight", §Restrições e verificação).
#include "tp_shard.h"
#include "tp_kernels.h"

#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <fcntl.h>
#include <unistd.h>
#include <algorithm>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

struct tp_block_shard {
  tp_block_config cfg;
  int device;
  size_t es;        // element size of activations and weights
  int64_t D, Dr, Fr, Hr, d;
  bool attn, mlp, swiglu;
  int64_t n_up;     // rows of the MLP in-projection slice: Fr, or 2 Fr with SwiGLU
  int64_t n_col;    // rows of the packed colwise weight: 3 Dr (attention) + n_up (MLP)
  int64_t up_row0;  // first row of W_up_r in it
  int64_t k_row;    // columns of the packed rowwise weight: Dr (attention) + Fr (MLP)
  int64_t dn_col0;  // first column of W_dn_r in it
  void* w_col;      // [n_col, D]      = [W_q[R_r]; W_k[R_r]; W_v[R_r]; W_up[C_r]]
                    //   SwiGLU: the MLP part is W_gate[C_r] and W_up[C_r] interleaved
                    //   in blocks of 32 rows: gate 0-31, up 0-31, gate 32-63, ...
  float* b_col;     // [n_col] fp32, the biases in the same row order
  void* w_row;      // [D, k_row]      = [W_o[:, R_r] | W_dn[:, C_r]]
  bool mod;
  int64_t mod_in, mod_out, mod_kr;  // modulation projection: K, N, K_r = K / P
  void* w_mod;      // [mod_out, mod_kr] = W_mod[:, M_r]
};

namespace {

thread_local std::string g_detail;

tp_status fail(tp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

tp_status hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? TP_ERR_OOM : TP_ERR_HIP, "%s: %s", what,
              hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A row-major device matrix argument: non-NULL, 16-byte aligned, ld >= width,
// every row start 16-byte aligned.
tp_status check_matrix(const char* name, const void* p, int64_t ld, int64_t width, size_t es) {
  if (!p) return fail(TP_ERR_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(TP_ERR_ARG, "%s is not 16-byte aligned", name);
  if (ld < width) return fail(TP_ERR_ARG, "ld of %s (%lld) < width %lld", name, (long long)ld,
                              (long long)width);
  if ((ld * (int64_t)es) % 16) return fail(TP_ERR_ARG, "ld of %s (%lld) is not a multiple of 16 bytes",
                                           name, (long long)ld);
  return TP_OK;
}

bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + b_bytes && pb < pa + a_bytes;
}

int64_t span_bytes(int64_t rows, int64_t ld, int64_t width, size_t es) {
  return rows <= 0 ? 0 : ((rows - 1) * ld + width) * (int64_t)es;
}

tp_status check_shard(const tp_block_shard* s) {
  if (!s) return fail(TP_ERR_ARG, "shard is NULL");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != s->device)
    return fail(TP_ERR_ARG, "current device %d is not the shard's device %d", dev, s->device);
  return TP_OK;
}

tp_status check_tokens(int64_t tokens) {
  if (tokens < 0) return fail(TP_ERR_ARG, "tokens (%lld) < 0", (long long)tokens);
  if (tokens > INT32_MAX) return fail(TP_ERR_UNSUPPORTED, "tokens (%lld) > 2^31-1", (long long)tokens);
  return TP_OK;
}

void free_shard(tp_block_shard* s) {
  if (!s) return;
  if (s->w_col) (void)hipFree(s->w_col);
  if (s->b_col) (void)hipFree(s->b_col);
  if (s->w_row) (void)hipFree(s->w_row);
  if (s->w_mod) (void)hipFree(s->w_mod);
  delete s;
}

tp_status launch(const tpk::GemmProblem& p, const tpk::GemmEpilogue& ep, tpk::OutKind kind,
                 tp_dtype dt, hipStream_t stream) {
  const hipError_t e = dt == TP_BF16 ? tpk::launch_gemm_bf16(p, ep, kind, stream)
                                     : tpk::launch_gemm_f32(p, ep, kind, stream);
  if (e != hipSuccess) return hip_fail(e, "GEMM launch");
  return TP_OK;
}

// A rowwise partial (no bias, fp32 out): the few-row bf16 kernel when the
// input has at most 64 rows, else the GEMM.
tp_status rowwise(const tpk::GemmProblem& p, float* partial, int64_t ldp, bool accumulate,
                  tp_dtype dt, hipStream_t stream) {
  if (dt == TP_BF16 && tpk::skinny_bf16_fits(p)) {
    const hipError_t e = tpk::launch_skinny_bf16(p, partial, ldp, accumulate, stream);
    if (e != hipSuccess) return hip_fail(e, "rowwise launch");
    return TP_OK;
  }
  const tpk::GemmEpilogue ep{nullptr, p.N, tpk::Act::NONE, p.N, partial, ldp, nullptr, 0};
  return launch(p, ep, accumulate ? tpk::OutKind::F32_ACC : tpk::OutKind::F32_STORE, dt, stream);
}

// Colwise GEMM over weight rows [row0, row0 + n_w) of the packed slice:
// activation `act` on GEMM columns >= act_from, output columns < split to y0,
// the rest to y1 (see tpk::GemmEpilogue).
tp_status colwise(const tp_block_shard* s, int64_t tokens, const void* x, int64_t ldx, int64_t row0,
                  int64_t n_w, tpk::Act act, int act_from, int split, void* y0, int64_t ld0,
                  void* y1, int64_t ld1, hipStream_t stream) {
  const tpk::GemmProblem p{x, ldx, static_cast<const char*>(s->w_col) + row0 * s->D * s->es, s->D,
                           (int)tokens, (int)n_w, (int)s->D};
  const tpk::GemmEpilogue ep{s->b_col + row0, act_from, act, split, y0, ld0, y1, ld1};
  return launch(p, ep, s->cfg.dtype == TP_BF16 ? tpk::OutKind::BF16 : tpk::OutKind::F32_STORE,
                s->cfg.dtype, stream);
}

constexpr int kReadThreads = 8;

// Where the unsharded weights come from.  Each weight is a row-major array;
// copy2d moves `rows` rows of `width` bytes, row i starting at byte
// off0 + i * pitch of that weight, to device rows of `dst_pitch` bytes.
enum WeightId { W_Q, W_K, W_V, B_Q, B_K, B_V, W_O, W_UP, B_UP, W_DOWN, W_MOD, kNumWeights };

struct WeightSource {
  virtual ~WeightSource() = default;
  virtual bool present(int which) const = 0;
  virtual tp_status open() = 0;      // before any device work: files exist
  virtual tp_status begin() = 0;     // after the device allocations
  virtual tp_status copy2d(int which, int64_t off0, int64_t pitch, int64_t width, int64_t rows,
                           char* dst, int64_t dst_pitch) = 0;
  virtual tp_status read(int which, int64_t off, int64_t bytes, void* host) = 0;
  virtual tp_status finish() { return TP_OK; }
  virtual void drain() {}  // wait for copies in flight (error path), keeping the error detail
};

// Caller's host arrays (tp_block_shard_create).
struct HostSource final : WeightSource {
  const void* p[kNumWeights];
  explicit HostSource(const tp_block_weights& w)
      : p{w.w_q, w.w_k, w.w_v, w.b_q, w.b_k, w.b_v, w.w_o, w.w_up, w.b_up, w.w_down, w.w_mod} {}
  bool present(int which) const override { return p[which] != nullptr; }
  tp_status open() override { return TP_OK; }
  tp_status begin() override { return TP_OK; }
  tp_status copy2d(int which, int64_t off0, int64_t pitch, int64_t width, int64_t rows, char* dst,
                   int64_t dst_pitch) override {
    const hipError_t e = hipMemcpy2D(dst, (size_t)dst_pitch, static_cast<const char*>(p[which]) + off0,
                                     (size_t)pitch, (size_t)width, (size_t)rows, hipMemcpyHostToDevice);
    return e == hipSuccess ? TP_OK : hip_fail(e, "weight slice upload");
  }
  tp_status read(int which, int64_t off, int64_t bytes, void* host) override {
    std::memcpy(host, static_cast<const char*>(p[which]) + off, (size_t)bytes);
    return TP_OK;
  }
};

// Raw weight files (tp_block_shard_load): only the rank's byte ranges are
// read, with pread, into one pinned staging buffer split in two halves; a
// half is copied to the device asynchronously while the next is read, so host
// memory stays at the staging size whatever the weights' size.  A half is
// filled by up to kReadThreads threads (one copy from the page cache per
// thread is what limits a single reader).
struct FileSource final : WeightSource {
  tp_weight_file f[kNumWeights];
  int fd[kNumWeights];
  int64_t staging_bytes;
  char* staging = nullptr;
  hipStream_t stream = nullptr;
  hipEvent_t done[2] = {nullptr, nullptr};
  bool busy[2] = {false, false};
  int half = 0;

  FileSource(const tp_block_weight_files& w, int64_t staging)
      : f{w.w_q, w.w_k, w.w_v, w.b_q, w.b_k, w.b_v, w.w_o, w.w_up, w.b_up, w.w_down, w.w_mod},
        staging_bytes(staging) {
    for (int& x : fd) x = -1;
  }
  ~FileSource() override {
    for (int i = 0; i < 2; ++i)
      if (done[i]) {
        (void)hipEventSynchronize(done[i]);
        (void)hipEventDestroy(done[i]);
      }
    if (stream) (void)hipStreamDestroy(stream);
    if (staging) (void)hipHostFree(staging);
    for (int x : fd)
      if (x >= 0) close(x);
  }
  bool present(int which) const override { return f[which].path != nullptr; }
  tp_status open() override {
    for (int i = 0; i < kNumWeights; ++i) {
      if (!f[i].path) continue;
      if (f[i].offset < 0) return fail(TP_ERR_ARG, "negative file offset for weight %d", i);
      fd[i] = ::open(f[i].path, O_RDONLY);
      if (fd[i] < 0) return fail(TP_ERR_IO, "cannot open %s: %s", f[i].path, strerror(errno));
    }
    return TP_OK;
  }
  tp_status begin() override {
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&staging), (size_t)staging_bytes,
                                 hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "staging buffer");
    if ((e = hipStreamCreate(&stream)) != hipSuccess) return hip_fail(e, "staging stream");
    for (int i = 0; i < 2; ++i)
      if ((e = hipEventCreateWithFlags(&done[i], hipEventDisableTiming)) != hipSuccess)
        return hip_fail(e, "staging event");
    return TP_OK;
  }
  // Reads [off, off + bytes) of weight `which`: 0, or -errno, or 1 if the file ends first.
  int read_range(int which, int64_t off, int64_t bytes, char* dst) const {
    int64_t got = 0;
    while (got < bytes) {
      const ssize_t n = ::pread(fd[which], dst + got, (size_t)(bytes - got), f[which].offset + off + got);
      if (n < 0 && errno == EINTR) continue;
      if (n < 0) return -errno;
      if (n == 0) return 1;
      got += n;
    }
    return 0;
  }
  tp_status report(int which, int rc, int64_t end) const {
    if (rc == 0) return TP_OK;
    if (rc > 0)
      return fail(TP_ERR_IO, "%s is too short: need byte %lld", f[which].path,
                  (long long)(f[which].offset + end));
    return fail(TP_ERR_IO, "read of %s failed: %s", f[which].path, strerror(-rc));
  }
  tp_status pread_all(int which, int64_t off, int64_t bytes, char* dst) {
    return report(which, read_range(which, off, bytes, dst), off + bytes);
  }
  // `n` row segments of `width` bytes, segment j at off0 + j * pitch, packed
  // into dst, read by up to kReadThreads threads.
  tp_status read_rows(int which, int64_t off0, int64_t pitch, int64_t width, int64_t n, char* dst) {
    const int64_t bytes = n * width;
    const int nt = (int)std::min<int64_t>(kReadThreads, std::max<int64_t>(1, bytes >> 22));
    std::vector<int> rc(nt, 0);
    auto work = [&](int t) {
      if (pitch == width) {  // one contiguous range: split it
        const int64_t a = bytes * t / nt, b = bytes * (t + 1) / nt;
        rc[t] = read_range(which, off0 + a, b - a, dst + a);
      } else {
        for (int64_t j = n * t / nt; j < n * (t + 1) / nt && rc[t] == 0; ++j)
          rc[t] = read_range(which, off0 + j * pitch, width, dst + j * width);
      }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < nt; ++t) pool.emplace_back(work, t);
    work(0);
    for (auto& th : pool) th.join();
    for (int t = 0; t < nt; ++t)
      if (rc[t]) return report(which, rc[t], off0 + (n - 1) * pitch + width);
    return TP_OK;
  }
  // The next free staging half (waits for its previous copy to finish).
  tp_status take(char** buf) {
    half ^= 1;
    if (busy[half]) {
      const hipError_t e = hipEventSynchronize(done[half]);
      if (e != hipSuccess) return hip_fail(e, "staging copy");
      busy[half] = false;
    }
    *buf = staging + half * (staging_bytes / 2);
    return TP_OK;
  }
  tp_status send(const char* buf, int64_t width, int64_t rows, char* dst, int64_t dst_pitch) {
    hipError_t e = hipMemcpy2DAsync(dst, (size_t)dst_pitch, buf, (size_t)width, (size_t)width,
                                    (size_t)rows, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipEventRecord(done[half], stream);
    if (e != hipSuccess) return hip_fail(e, "staging copy");
    busy[half] = true;
    return TP_OK;
  }
  tp_status copy2d(int which, int64_t off0, int64_t pitch, int64_t width, int64_t rows, char* dst,
                   int64_t dst_pitch) override {
    const int64_t cap = staging_bytes / 2;
    tp_status st = TP_OK;
    if (width > cap) {  // long rows: stream each row in pieces
      for (int64_t i = 0; i < rows && st == TP_OK; ++i)
        for (int64_t c = 0; c < width && st == TP_OK; c += cap) {
          const int64_t n = width - c < cap ? width - c : cap;
          char* buf;
          if ((st = take(&buf)) == TP_OK && (st = read_rows(which, off0 + i * pitch + c, n, n, 1, buf)) == TP_OK)
            st = send(buf, n, 1, dst + i * dst_pitch + c, n);
        }
      return st;
    }
    const int64_t per = cap / width;  // rows per staging half
    for (int64_t i = 0; i < rows && st == TP_OK; i += per) {
      const int64_t n = rows - i < per ? rows - i : per;
      char* buf;
      if ((st = take(&buf)) != TP_OK) break;
      st = read_rows(which, off0 + i * pitch, pitch, width, n, buf);
      if (st == TP_OK) st = send(buf, width, n, dst + i * dst_pitch, dst_pitch);
    }
    return st;
  }
  tp_status read(int which, int64_t off, int64_t bytes, void* host) override {
    return pread_all(which, off, bytes, static_cast<char*>(host));
  }
  tp_status finish() override {
    const hipError_t e = hipStreamSynchronize(stream);
    return e == hipSuccess ? TP_OK : hip_fail(e, "staging copy");
  }
  void drain() override {
    if (stream) (void)hipStreamSynchronize(stream);
  }
};

constexpr int64_t kMinStaging = (int64_t)1 << 20;

// fp32 copy of bias elements [from, from + n) into dst[at..]; absent = zero.
tp_status read_bias(WeightSource& src, int which, std::vector<float>& dst, int64_t at, int64_t from,
                    int64_t n, tp_dtype dt) {
  if (!src.present(which)) return TP_OK;
  if (dt == TP_F32) return src.read(which, from * 4, n * 4, dst.data() + at);
  std::vector<uint16_t> b((size_t)n);
  tp_status st = src.read(which, from * 2, n * 2, b.data());
  if (st != TP_OK) return st;
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t bits = (uint32_t)b[i] << 16;  // exact bf16 -> fp32 widening
    std::memcpy(&dst[at + i], &bits, 4);
  }
  return TP_OK;
}

// Validation, allocation and slice upload shared by create (host arrays) and
// load (files): every check runs before any weight byte is read.
tp_status create_from(const tp_block_config* cfg, WeightSource& src, int64_t w_ld_o,
                      int64_t w_ld_down, tp_block_shard** out) {
  if (cfg->dtype != TP_F32 && cfg->dtype != TP_BF16)
    return fail(TP_ERR_ARG, "unknown dtype %d", (int)cfg->dtype);
  if (cfg->mlp_act != TP_MLP_GELU_TANH && cfg->mlp_act != TP_MLP_SWIGLU)
    return fail(TP_ERR_ARG, "unknown mlp_act %d", (int)cfg->mlp_act);
  const int64_t P = cfg->tp_degree, r = cfg->rank, D = cfg->hidden, H = cfg->num_heads,
                d = cfg->head_dim, F = cfg->ffn;
  if (P < 1 || r < 0 || r >= P)
    return fail(TP_ERR_ARG, "rank %lld not in [0, tp_degree=%lld)", (long long)r, (long long)P);
  const int64_t Mi = cfg->mod_in, Mo = cfg->mod_out;
  if (D <= 0 || H < 0 || F < 0 || Mi < 0 || Mo < 0) return fail(TP_ERR_ARG, "sizes must be positive");
  if ((Mi > 0) != (Mo > 0))
    return fail(TP_ERR_ARG, "mod_in and mod_out must both be zero or both positive");
  if (H == 0 && F == 0 && Mo == 0)
    return fail(TP_ERR_ARG, "neither attention (num_heads), MLP (ffn) nor modulation (mod_out)");
  if (H > 0 && d <= 0) return fail(TP_ERR_ARG, "head_dim must be positive");
  if (H > 0) {
    if (H * d != D)
      return fail(TP_ERR_DIVISIBILITY, "num_heads*head_dim = %lld != hidden %lld",
                  (long long)(H * d), (long long)D);
    if (H % P)
      return fail(TP_ERR_DIVISIBILITY, "tp_degree %lld does not divide num_heads %lld",
                  (long long)P, (long long)H);
    if (D % P)
      return fail(TP_ERR_DIVISIBILITY, "tp_degree %lld does not divide the Q/K/V blocks (%lld)",
                  (long long)P, (long long)D);
  }
  if (F % P)
    return fail(TP_ERR_DIVISIBILITY, "tp_degree %lld does not divide ffn %lld", (long long)P,
                (long long)F);
  if (Mi % P)
    return fail(TP_ERR_DIVISIBILITY, "tp_degree %lld does not divide the modulation input %lld",
                (long long)P, (long long)Mi);
  const int64_t Dr = H > 0 ? D / P : 0, Fr = F / P;
  const bool swiglu = F > 0 && cfg->mlp_act == TP_MLP_SWIGLU;
  if (D % 8 || Dr % 8 || Fr % 8)
    return fail(TP_ERR_UNSUPPORTED, "hidden, hidden/tp and ffn/tp must be multiples of 8");
  if ((Mi / P) % 8 || Mo % 8)
    return fail(TP_ERR_UNSUPPORTED, "mod_in/tp and mod_out must be multiples of 8");
  if (swiglu && Fr % 32)
    return fail(TP_ERR_UNSUPPORTED, "SwiGLU needs ffn/tp (%lld) to be a multiple of 32",
                (long long)Fr);
  if (H > 0 && (!src.present(W_Q) || !src.present(W_K) || !src.present(W_V) || !src.present(W_O)))
    return fail(TP_ERR_ARG, "attention configured but w_q/w_k/w_v/w_o missing");
  if (F > 0 && (!src.present(W_UP) || !src.present(W_DOWN)))
    return fail(TP_ERR_ARG, "MLP configured but w_up/w_down missing");
  if (Mo > 0 && !src.present(W_MOD)) return fail(TP_ERR_ARG, "modulation configured but w_mod missing");
  const int64_t ld_o = w_ld_o ? w_ld_o : H * d, ld_dn = w_ld_down ? w_ld_down : F;
  if (H > 0 && ld_o < H * d)
    return fail(TP_ERR_ARG, "ld_o (%lld) < num_heads*head_dim (%lld)", (long long)ld_o,
                (long long)(H * d));
  if (F > 0 && ld_dn < F)
    return fail(TP_ERR_ARG, "ld_down (%lld) < ffn (%lld)", (long long)ld_dn, (long long)F);

  tp_status st = src.open();
  if (st != TP_OK) return st;

  tp_block_shard* s = new tp_block_shard();
  s->cfg = *cfg;
  s->es = cfg->dtype == TP_BF16 ? 2 : 4;
  s->D = D; s->Dr = Dr; s->Fr = Fr; s->Hr = H / P; s->d = d;
  s->attn = H > 0; s->mlp = F > 0; s->swiglu = swiglu;
  s->up_row0 = 3 * Dr;
  s->n_up = swiglu ? 2 * Fr : Fr;
  s->n_col = 3 * Dr + s->n_up;
  s->dn_col0 = Dr;
  s->k_row = Dr + Fr;
  s->mod = Mo > 0; s->mod_in = Mi; s->mod_out = Mo; s->mod_kr = Mi / P;
  hipError_t e = hipGetDevice(&s->device);
  if (e != hipSuccess) { free_shard(s); return hip_fail(e, "hipGetDevice"); }

  const size_t es = s->es;
  const bool block = s->attn || s->mlp;
  if (block && ((e = hipMalloc(&s->w_col, (size_t)(s->n_col * D) * es)) != hipSuccess ||
                (e = hipMalloc(reinterpret_cast<void**>(&s->b_col), (size_t)s->n_col * sizeof(float))) != hipSuccess ||
                (e = hipMalloc(&s->w_row, (size_t)(D * s->k_row) * es)) != hipSuccess)) {
    free_shard(s);
    return hip_fail(e, "hipMalloc of the weight slices");
  }
  if (s->mod && (e = hipMalloc(&s->w_mod, (size_t)(Mo * s->mod_kr) * es)) != hipSuccess) {
    free_shard(s);
    return hip_fail(e, "hipMalloc of the modulation slice");
  }

  if ((st = src.begin()) != TP_OK) {
    free_shard(s);
    return st;
  }
  // Colwise slices: contiguous blocks of dim-0 rows, one per packed block.
  std::vector<float> bias((size_t)s->n_col, 0.0f);
  char* wc = static_cast<char*>(s->w_col);
  const int64_t row_bytes = D * (int64_t)es;
  auto put_rows = [&](int which, int64_t src_row0, int64_t nrows, int64_t dst_row0) {
    return src.copy2d(which, src_row0 * row_bytes, nrows * row_bytes, nrows * row_bytes, 1,
                      wc + dst_row0 * row_bytes, nrows * row_bytes);
  };
  if (s->attn) {
    const int ws[3] = {W_Q, W_K, W_V}, bs[3] = {B_Q, B_K, B_V};
    for (int b = 0; b < 3 && st == TP_OK; ++b) {
      st = put_rows(ws[b], r * Dr, Dr, b * Dr);
      if (st == TP_OK) st = read_bias(src, bs[b], bias, b * Dr, r * Dr, Dr, cfg->dtype);
    }
  }
  if (st == TP_OK && s->mlp && !swiglu) {
    st = put_rows(W_UP, r * Fr, Fr, s->up_row0);
    if (st == TP_OK) st = read_bias(src, B_UP, bias, s->up_row0, r * Fr, Fr, cfg->dtype);
  }
  if (st == TP_OK && swiglu) {
    // [1, 1] blocks: the rank's gate rows C_r and up rows F + C_r, stored as
    // alternating 32-row blocks so the GEMM epilogue finds a gate column and
    // its up column in neighbouring 32-column MFMA tiles.
    const int64_t blk = 32, nblk = Fr / blk;
    for (int half = 0; half < 2 && st == TP_OK; ++half) {
      const int64_t src_row0 = half * F + r * Fr;
      st = src.copy2d(W_UP, src_row0 * row_bytes, blk * row_bytes, blk * row_bytes, nblk,
                      wc + (s->up_row0 + half * blk) * row_bytes, 2 * blk * row_bytes);
      for (int64_t b = 0; b < nblk && st == TP_OK; ++b)
        st = read_bias(src, B_UP, bias, s->up_row0 + 2 * blk * b + half * blk, src_row0 + blk * b,
                       blk, cfg->dtype);
    }
  }
  if (st == TP_OK && block) {
    const hipError_t e2 = hipMemcpy(s->b_col, bias.data(), bias.size() * sizeof(float),
                                    hipMemcpyHostToDevice);
    if (e2 != hipSuccess) st = hip_fail(e2, "bias upload");
  }
  // Rowwise slices: dim-1 column blocks, copied as strided 2-D regions.
  char* wr = static_cast<char*>(s->w_row);
  const int64_t dpitch = s->k_row * (int64_t)es;
  if (st == TP_OK && s->attn)
    st = src.copy2d(W_O, r * Dr * (int64_t)es, ld_o * (int64_t)es, Dr * (int64_t)es, D, wr, dpitch);
  if (st == TP_OK && s->mlp)
    st = src.copy2d(W_DOWN, r * Fr * (int64_t)es, ld_dn * (int64_t)es, Fr * (int64_t)es, D,
                    wr + s->dn_col0 * (int64_t)es, dpitch);
  // Modulation slice ("rowwise_split_input"): dim-1 columns M_r.
  if (st == TP_OK && s->mod)
    st = src.copy2d(W_MOD, r * s->mod_kr * (int64_t)es, Mi * (int64_t)es, s->mod_kr * (int64_t)es,
                    Mo, static_cast<char*>(s->w_mod), s->mod_kr * (int64_t)es);
  if (st == TP_OK) st = src.finish();
  if (st != TP_OK) {
    src.drain();
    free_shard(s);
    return st;
  }
  *out = s;
  return TP_OK;
}


}  // namespace

extern "C" {

TP_API tp_status tp_block_shard_create(const tp_block_config* cfg, const tp_block_weights* w,
                                       tp_block_shard** out) {
  if (!out) return fail(TP_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg || !w) return fail(TP_ERR_ARG, "config or weights is NULL");
  HostSource src(*w);
  return create_from(cfg, src, w->ld_o, w->ld_down, out);
}

TP_API tp_status tp_block_shard_load(const tp_block_config* cfg, const tp_block_weight_files* files,
                                     int64_t staging_bytes, tp_block_shard** out) {
  if (!out) return fail(TP_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg || !files) return fail(TP_ERR_ARG, "config or files is NULL");
  if (staging_bytes < kMinStaging)
    return fail(TP_ERR_ARG, "staging_bytes (%lld) < %lld", (long long)staging_bytes,
                (long long)kMinStaging);
  FileSource src(*files, staging_bytes);
  return create_from(cfg, src, files->ld_o, files->ld_down, out);
}

TP_API void tp_block_shard_destroy(tp_block_shard* shard) { free_shard(shard); }

TP_API tp_status tp_colwise_linear(tp_block_shard* s, tp_layer layer, int64_t tokens, const void* x,
                                   int64_t ldx, void* y, int64_t ldy, void* stream) {
  tp_status st = check_shard(s);
  if (st != TP_OK) return st;
  int64_t row0, n, n_w;  // first weight row, output width, weight rows (GEMM N)
  tpk::Act act;
  if (layer == TP_QKV) {
    if (!s->attn) return fail(TP_ERR_ARG, "TP_QKV: shard has no attention layers");
    row0 = 0; n = n_w = 3 * s->Dr; act = tpk::Act::NONE;
  } else if (layer == TP_MLP_UP) {
    if (!s->mlp) return fail(TP_ERR_ARG, "TP_MLP_UP: shard has no MLP layers");
    row0 = s->up_row0; n = s->Fr; n_w = s->n_up;
    act = s->swiglu ? tpk::Act::SWIGLU : tpk::Act::GELU_TANH;
  } else {
    return fail(TP_ERR_ARG, "layer %d is not colwise (TP_QKV or TP_MLP_UP)", (int)layer);
  }
  if ((st = check_tokens(tokens)) != TP_OK) return st;
  if ((st = check_matrix("x", x, ldx, s->D, s->es)) != TP_OK) return st;
  if ((st = check_matrix("y", y, ldy, n, s->es)) != TP_OK) return st;
  if (tokens == 0) return TP_OK;
  return colwise(s, tokens, x, ldx, row0, n_w, act, 0, (int)n, y, ldy, nullptr, 0,
                 static_cast<hipStream_t>(stream));
}

TP_API tp_status tp_colwise_qkv_up(tp_block_shard* s, int64_t tokens, const void* x, int64_t ldx,
                                   void* qkv, int64_t ldqkv, void* h, int64_t ldh, void* stream) {
  tp_status st = check_shard(s);
  if (st != TP_OK) return st;
  if (!s->attn || !s->mlp) return fail(TP_ERR_ARG, "tp_colwise_qkv_up needs attention and MLP");
  if ((st = check_tokens(tokens)) != TP_OK) return st;
  if ((st = check_matrix("x", x, ldx, s->D, s->es)) != TP_OK) return st;
  if ((st = check_matrix("qkv", qkv, ldqkv, 3 * s->Dr, s->es)) != TP_OK) return st;
  if ((st = check_matrix("h", h, ldh, s->Fr, s->es)) != TP_OK) return st;
  if (tokens == 0) return TP_OK;
  if (overlap(qkv, span_bytes(tokens, ldqkv, 3 * s->Dr, s->es), h, span_bytes(tokens, ldh, s->Fr, s->es)))
    return fail(TP_ERR_ARG, "qkv and h overlap");
  const int split = (int)(3 * s->Dr);
  const hipStream_t st_ = static_cast<hipStream_t>(stream);
  if (s->swiglu && split % 64) {
    // SwiGLU pairs need the MLP rows to start on a 64-column boundary of the
    // GEMM; otherwise the two projections run as two launches.
    if ((st = colwise(s, tokens, x, ldx, 0, split, tpk::Act::NONE, split, split, qkv, ldqkv,
                      nullptr, 0, st_)) != TP_OK)
      return st;
    return colwise(s, tokens, x, ldx, s->up_row0, s->n_up, tpk::Act::SWIGLU, 0, (int)s->Fr, h, ldh,
                   nullptr, 0, st_);
  }
  return colwise(s, tokens, x, ldx, 0, s->n_col,
                 s->swiglu ? tpk::Act::SWIGLU : tpk::Act::GELU_TANH, split, split, qkv, ldqkv, h,
                 ldh, st_);
}

TP_API tp_status tp_attn_heads(tp_block_shard* s, int64_t tokens, const void* qkv, int64_t ldqkv,
                               void* o, int64_t ldo, void* stream) {
  tp_status st = check_shard(s);
  if (st != TP_OK) return st;
  if (!s->attn) return fail(TP_ERR_ARG, "shard has no attention layers");
  if (s->cfg.dtype != TP_BF16) return fail(TP_ERR_UNSUPPORTED, "attention is built for bf16 only");
  if (s->d != 128) return fail(TP_ERR_UNSUPPORTED, "attention is built for head_dim 128 only");
  if ((st = check_tokens(tokens)) != TP_OK) return st;
  if ((st = check_matrix("qkv", qkv, ldqkv, 3 * s->Dr, s->es)) != TP_OK) return st;
  if ((st = check_matrix("o", o, ldo, s->Dr, s->es)) != TP_OK) return st;
  if (tokens == 0) return TP_OK;
  if (overlap(qkv, span_bytes(tokens, ldqkv, 3 * s->Dr, s->es), o, span_bytes(tokens, ldo, s->Dr, s->es)))
    return fail(TP_ERR_ARG, "o overlaps qkv");
  const hipError_t e = tpk::launch_attn_fwd_bf16_d128(qkv, ldqkv, o, ldo, (int)tokens, (int)s->Hr,
                                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return TP_OK;
}

// Queries of q_qkv against the keys and values of kv_qkv, the keys cut into
// n_splits balanced ranges in one launch; range z writes its normalised fp32
// output at o + z o_stride and its log-sum-exp at lse + z lse_stride.
// tp_attn_heads_block (one range), tp_attn_heads_split (q_qkv == kv_qkv) and
// tp_attn_heads_block_split share it.
static tp_status attn_parts(tp_block_shard* s, int64_t q_tokens, const void* q_qkv, int64_t ldq,
                            int64_t kv_tokens, const void* kv_qkv, int64_t ldkv, int32_t n_splits,
                            float* o, int64_t ldo, int64_t o_stride, float* lse, int64_t ld_lse,
                            int64_t lse_stride, void* stream) {
  tp_status st = check_shard(s);
  if (st != TP_OK) return st;
  if (!s->attn) return fail(TP_ERR_ARG, "shard has no attention layers");
  if (s->cfg.dtype != TP_BF16) return fail(TP_ERR_UNSUPPORTED, "attention is built for bf16 only");
  if (s->d != 128) return fail(TP_ERR_UNSUPPORTED, "attention is built for head_dim 128 only");
  if ((st = check_tokens(q_tokens)) != TP_OK) return st;
  if ((st = check_tokens(kv_tokens)) != TP_OK) return st;
  if (n_splits < 1) return fail(TP_ERR_ARG, "n_splits (%d) < 1", n_splits);
  if (n_splits > tpk::kMaxMergeParts)
    return fail(TP_ERR_UNSUPPORTED, "n_splits (%d) > %d", n_splits, tpk::kMaxMergeParts);
  const int64_t Dr = s->Dr, Hr = s->Hr;
  if ((st = check_matrix("q_qkv", q_qkv, ldq, Dr, s->es)) != TP_OK) return st;
  if ((st = check_matrix("kv_qkv", kv_qkv, ldkv, 3 * Dr, s->es)) != TP_OK) return st;
  if ((st = check_matrix("o", o, ldo, Dr, sizeof(float))) != TP_OK) return st;
  if (o_stride % 4) return fail(TP_ERR_ARG, "the o part stride must keep parts 16-byte aligned");
  if (!lse) return fail(TP_ERR_ARG, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(TP_ERR_ARG, "lse is not 4-byte aligned");
  if (ld_lse < Hr) return fail(TP_ERR_ARG, "ld_lse (%lld) < local heads %lld", (long long)ld_lse,
                               (long long)Hr);
  if (q_tokens == 0) return TP_OK;
  if (kv_tokens < n_splits)
    return fail(TP_ERR_ARG, n_splits == 1 ? "kv_tokens must be >= 1" : "fewer keys than key splits");
  const int64_t ob = span_bytes(q_tokens, ldo, Dr, sizeof(float));
  const int64_t lb = span_bytes(q_tokens, ld_lse, Hr, sizeof(float));
  if (n_splits > 1 && (o_stride * (int64_t)sizeof(float) < ob || lse_stride * (int64_t)sizeof(float) < lb))
    return fail(TP_ERR_ARG, "part strides shorter than one part (parts would overlap)");
  const int64_t o_all = (n_splits - 1) * o_stride * (int64_t)sizeof(float) + ob;
  const int64_t l_all = (n_splits - 1) * lse_stride * (int64_t)sizeof(float) + lb;
  const int64_t qb = span_bytes(q_tokens, ldq, Dr, s->es);
  const int64_t kb = span_bytes(kv_tokens, ldkv, 3 * Dr, s->es);
  if (overlap(o, o_all, q_qkv, qb) || overlap(o, o_all, kv_qkv, kb) || overlap(lse, l_all, q_qkv, qb) ||
      overlap(lse, l_all, kv_qkv, kb) || overlap(o, o_all, lse, l_all))
    return fail(TP_ERR_ARG, "o / lse parts overlap each other or the inputs");
  const char* kv = static_cast<const char*>(kv_qkv);
  const tpk::AttnBlockArgs a{q_qkv, ldq, kv + Dr * s->es, kv + 2 * Dr * s->es, ldkv,
                             (int)q_tokens, (int)kv_tokens, (int)Hr, o, ldo, lse, ld_lse,
                             n_splits, o_stride, lse_stride};
  const hipError_t e = tpk::launch_attn_block_bf16_d128(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return TP_OK;
}

TP_API tp_status tp_attn_heads_block(tp_block_shard* s, int64_t q_tokens, const void* q_qkv,
                                     int64_t ldq, int64_t kv_tokens, const void* kv_qkv,
                                     int64_t ldkv, float* o, int64_t ldo, float* lse,
                                     int64_t ld_lse, void* stream) {
  return attn_parts(s, q_tokens, q_qkv, ldq, kv_tokens, kv_qkv, ldkv, 1, o, ldo, 0, lse, ld_lse, 0,
                    stream);
}

TP_API tp_status tp_attn_heads_block_split(tp_block_shard* s, int64_t q_tokens, const void* q_qkv,
                                           int64_t ldq, int64_t kv_tokens, const void* kv_qkv,
                                           int64_t ldkv, int32_t n_splits, float* o_parts,
                                           int64_t ldo, int64_t o_part_stride, float* lse_parts,
                                           int64_t ld_lse, int64_t lse_part_stride, void* stream) {
  return attn_parts(s, q_tokens, q_qkv, ldq, kv_tokens, kv_qkv, ldkv, n_splits, o_parts, ldo,
                    o_part_stride, lse_parts, ld_lse, lse_part_stride, stream);
}

TP_API tp_status tp_attn_heads_split(tp_block_shard* s, int64_t tokens, const void* qkv,
                                     int64_t ldqkv, int32_t n_splits, float* o_parts, int64_t ldo,
                                     int64_t o_part_stride, float* lse_parts, int64_t ld_lse,
                                     int64_t lse_part_stride, void* stream) {
  return attn_parts(s, tokens, qkv, ldqkv, tokens, qkv, ldqkv, n_splits, o_parts, ldo, o_part_stride,
                    lse_parts, ld_lse, lse_part_stride, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free split attention: the partial outputs and log-sum-exps of
// the key ranges live in `scratch`, one file-scope device array per GPU,
// instead of caller buffers.  In host code `scratch` names a host-side stand-in
// for the array, not its device address: that is looked up once per device
// (with the device current) and kept in scratch_ptr.
static constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxScratchDevices];

tp_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(TP_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table covers", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return TP_OK;
}

}  // namespace

TP_API tp_status tp_attn_heads_split_noalloc(tp_block_shard* s, int64_t tokens, const void* qkv,
                                             int64_t ldqkv, int32_t n_splits, void* o, int64_t ldo,
                                             void* stream) {
  tp_status st = check_shard(s);
  if (st != TP_OK) return st;
  if (!s->attn) return fail(TP_ERR_ARG, "shard has no attention layers");
  if (s->cfg.dtype != TP_BF16) return fail(TP_ERR_UNSUPPORTED, "attention is built for bf16 only");
  if (s->d != 128) return fail(TP_ERR_UNSUPPORTED, "attention is built for head_dim 128 only");
  if ((st = check_tokens(tokens)) != TP_OK) return st;
  if (n_splits < 1) return fail(TP_ERR_ARG, "n_splits (%d) < 1", n_splits);
  if (n_splits > tpk::kMaxMergeParts)
    return fail(TP_ERR_UNSUPPORTED, "n_splits (%d) > %d", n_splits, tpk::kMaxMergeParts);
  const int64_t Dr = s->Dr, Hr = s->Hr;
  if ((st = check_matrix("qkv", qkv, ldqkv, 3 * Dr, s->es)) != TP_OK) return st;
  if ((st = check_matrix("o", o, ldo, Dr, s->es)) != TP_OK) return st;
  if (tokens == 0) return TP_OK;
  if (tokens < n_splits) return fail(TP_ERR_ARG, "fewer tokens than key splits");
  if (overlap(qkv, span_bytes(tokens, ldqkv, 3 * Dr, s->es), o, span_bytes(tokens, ldo, Dr, s->es)))
    return fail(TP_ERR_ARG, "o overlaps qkv");
  // parts, contiguous: n_splits x [tokens, D_r] fp32 outputs, then
  // n_splits x [tokens, H/P] fp32 log-sum-exps (D_r is a multiple of 128, so
  // every part starts 16-byte aligned)
  const int64_t o_part = tokens * Dr, l_part = tokens * Hr;
  const int64_t need = (int64_t)n_splits * (o_part + l_part) * (int64_t)sizeof(float);
  if (need > kScratchBytes)
    return fail(TP_ERR_ARG, "%d key splits of %lld tokens need %lld bytes of scratch; the maximum is %lld",
                n_splits, (long long)tokens, (long long)need, (long long)kScratchBytes);
  void* base = nullptr;
  if ((st = scratch_of_current_device(&base)) != TP_OK) return st;
  float* o_parts = static_cast<float*>(base);
  float* l_parts = o_parts + n_splits * o_part;
  const char* kv = static_cast<const char*>(qkv);
  const tpk::AttnBlockArgs a{qkv, ldqkv, kv + Dr * s->es, kv + 2 * Dr * s->es, ldqkv,
                             (int)tokens, (int)tokens, (int)Hr, o_parts, Dr, l_parts, Hr,
                             n_splits, o_part, l_part};
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = tpk::launch_attn_block_bf16_d128(a, hs);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  tpk::MergeArgs m{};
  for (int i = 0; i < n_splits; ++i) {
    m.o[i] = o_parts + i * o_part;
    m.lse[i] = l_parts + i * l_part;
  }
  m.n = n_splits;
  m.ldo_in = Dr;
  m.ld_lse_in = Hr;
  m.T = (int)tokens;
  m.heads = (int)Hr;
  m.head_dim = (int)s->d;
  m.out = o;
  m.out_bf16 = true;
  m.ldo = ldo;
  m.lse_out = nullptr;
  m.ld_lse_out = 0;
  e = tpk::launch_attn_merge(m, hs);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return TP_OK;
}

TP_API int32_t tp_attn_split_hint(const tp_block_shard* s, int64_t tokens) {
  if (!s || !s->attn || tokens < 1 || tokens > INT32_MAX) return 1;
  return tpk::attn_split_hint((int)tokens, (int)s->Hr);
}

TP_API tp_status tp_attn_merge(const float* const* o_parts, const float* const* lse_parts,
                               int32_t n_parts, int64_t ldo_parts, int64_t ld_lse_parts,
                               int64_t tokens, int64_t heads, int64_t head_dim, void* o,
                               int64_t ldo, tp_dtype o_dtype, float* lse_out, int64_t ld_lse_out,
                               void* stream) {
  if (!o_parts || !lse_parts) return fail(TP_ERR_ARG, "o_parts or lse_parts is NULL");
  if (n_parts < 1) return fail(TP_ERR_ARG, "n_parts (%d) < 1", n_parts);
  if (n_parts > tpk::kMaxMergeParts)
    return fail(TP_ERR_UNSUPPORTED, "n_parts (%d) > %d", n_parts, tpk::kMaxMergeParts);
  if (o_dtype != TP_F32 && o_dtype != TP_BF16) return fail(TP_ERR_ARG, "unknown o_dtype");
  tp_status st = check_tokens(tokens);
  if (st != TP_OK) return st;
  if (heads < 1 || head_dim < 4 || head_dim % 4)
    return fail(TP_ERR_ARG, "heads >= 1 and head_dim a positive multiple of 4 required");
  const int64_t W = heads * head_dim;
  // the merge grid's column blocks (256 threads of 4 dims each) must not exceed 65535
  if (W > (int64_t)65535 * 256 * 4)
    return fail(TP_ERR_UNSUPPORTED, "heads*head_dim (%lld) too large", (long long)W);
  if (ld_lse_parts < heads) return fail(TP_ERR_ARG, "ld_lse_parts < heads");
  tpk::MergeArgs a{};
  for (int i = 0; i < n_parts; ++i) {
    if ((st = check_matrix("o_parts[i]", o_parts[i], ldo_parts, W, sizeof(float))) != TP_OK) return st;
    if (!lse_parts[i] || (reinterpret_cast<uintptr_t>(lse_parts[i]) & 3u))
      return fail(TP_ERR_ARG, "lse_parts[%d] is NULL or not 4-byte aligned", i);
    a.o[i] = o_parts[i];
    a.lse[i] = lse_parts[i];
  }
  const size_t oes = o_dtype == TP_BF16 ? 2 : 4;
  if ((st = check_matrix("o", o, ldo, W, oes)) != TP_OK) return st;
  if (lse_out) {
    if (reinterpret_cast<uintptr_t>(lse_out) & 3u) return fail(TP_ERR_ARG, "lse_out not 4-byte aligned");
    if (ld_lse_out < heads) return fail(TP_ERR_ARG, "ld_lse_out < heads");
  }
  if (tokens == 0) return TP_OK;
  const int64_t ob = span_bytes(tokens, ldo, W, oes);
  const int64_t lb = lse_out ? span_bytes(tokens, ld_lse_out, heads, sizeof(float)) : 0;
  for (int i = 0; i < n_parts; ++i) {
    const int64_t pb = span_bytes(tokens, ldo_parts, W, sizeof(float));
    const int64_t qb = span_bytes(tokens, ld_lse_parts, heads, sizeof(float));
    if (overlap(o, ob, o_parts[i], pb) || overlap(o, ob, lse_parts[i], qb) ||
        (lse_out && (overlap(lse_out, lb, o_parts[i], pb) || overlap(lse_out, lb, lse_parts[i], qb))))
      return fail(TP_ERR_ARG, "the merged output overlaps part %d", i);
  }
  if (lse_out && overlap(o, ob, lse_out, lb)) return fail(TP_ERR_ARG, "o overlaps lse_out");
  a.n = n_parts;
  a.ldo_in = ldo_parts;
  a.ld_lse_in = ld_lse_parts;
  a.T = (int)tokens;
  a.heads = (int)heads;
  a.head_dim = (int)head_dim;
  a.out = o;
  a.out_bf16 = o_dtype == TP_BF16;
  a.ldo = ldo;
  a.lse_out = lse_out;
  a.ld_lse_out = ld_lse_out;
  const hipError_t e = tpk::launch_attn_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return TP_OK;
}

TP_API tp_status tp_rowwise_linear_partial(tp_block_shard* s, tp_layer layer, int64_t tokens,
                                           const void* x_local, int64_t ldx, float* partial,
                                           int64_t ldp, int accumulate, void* stream) {
  tp_status st = check_shard(s);
  if (st != TP_OK) return st;
  int64_t col0, k;
  if (layer == TP_ATTN_OUT) {
    if (!s->attn) return fail(TP_ERR_ARG, "TP_ATTN_OUT: shard has no attention layers");
    col0 = 0; k = s->Dr;
  } else if (layer == TP_MLP_DOWN) {
    if (!s->mlp) return fail(TP_ERR_ARG, "TP_MLP_DOWN: shard has no MLP layers");
    col0 = s->dn_col0; k = s->Fr;
  } else if (layer == TP_BLOCK_OUT) {
    if (!s->attn || !s->mlp) return fail(TP_ERR_ARG, "TP_BLOCK_OUT needs attention and MLP");
    col0 = 0; k = s->k_row;
  } else {
    return fail(TP_ERR_ARG, "layer %d is not rowwise", (int)layer);
  }
  if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "accumulate must be 0 or 1");
  if ((st = check_tokens(tokens)) != TP_OK) return st;
  if ((st = check_matrix("x_local", x_local, ldx, k, s->es)) != TP_OK) return st;
  if ((st = check_matrix("partial", partial, ldp, s->D, sizeof(float))) != TP_OK) return st;
  if (tokens == 0) return TP_OK;
  if (overlap(x_local, span_bytes(tokens, ldx, k, s->es), partial,
              span_bytes(tokens, ldp, s->D, sizeof(float))))
    return fail(TP_ERR_ARG, "partial overlaps x_local");
  const tpk::GemmProblem p{x_local, ldx, static_cast<const char*>(s->w_row) + col0 * s->es, s->k_row,
                           (int)tokens, (int)s->D, (int)k};
  return rowwise(p, partial, ldp, accumulate != 0, s->cfg.dtype, static_cast<hipStream_t>(stream));
}

TP_API tp_status tp_rowwise_split_input_partial(tp_block_shard* s, tp_layer layer, int64_t rows,
                                                const void* x_full, int64_t ldx, float* partial,
                                                int64_t ldp, int accumulate, void* stream) {
  tp_status st = check_shard(s);
  if (st != TP_OK) return st;
  const int64_t r = s->cfg.rank, HD = s->Dr * s->cfg.tp_degree, F = s->cfg.ffn;
  int64_t width, n;        // replicated input width, output width
  if (layer == TP_ADALN_MOD) {
    if (!s->mod) return fail(TP_ERR_ARG, "TP_ADALN_MOD: shard has no modulation projection");
    width = s->mod_in; n = s->mod_out;
  } else if (layer == TP_ATTN_OUT) {
    if (!s->attn) return fail(TP_ERR_ARG, "TP_ATTN_OUT: shard has no attention layers");
    width = HD; n = s->D;
  } else if (layer == TP_MLP_DOWN) {
    if (!s->mlp) return fail(TP_ERR_ARG, "TP_MLP_DOWN: shard has no MLP layers");
    width = F; n = s->D;
  } else if (layer == TP_BLOCK_OUT) {
    if (!s->attn || !s->mlp) return fail(TP_ERR_ARG, "TP_BLOCK_OUT needs attention and MLP");
    width = HD + F; n = s->D;
  } else {
    return fail(TP_ERR_ARG, "layer %d is not rowwise", (int)layer);
  }
  if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "accumulate must be 0 or 1");
  if ((st = check_tokens(rows)) != TP_OK) return st;
  if ((st = check_matrix("x_full", x_full, ldx, width, s->es)) != TP_OK) return st;
  if ((st = check_matrix("partial", partial, ldp, n, sizeof(float))) != TP_OK) return st;
  if (rows == 0) return TP_OK;
  if (overlap(x_full, span_bytes(rows, ldx, width, s->es), partial,
              span_bytes(rows, ldp, n, sizeof(float))))
    return fail(TP_ERR_ARG, "partial overlaps x_full");
  const char* x = static_cast<const char*>(x_full);
  const hipStream_t st_ = static_cast<hipStream_t>(stream);
  const tp_dtype dt = s->cfg.dtype;
  if (layer == TP_ADALN_MOD) {
    const tpk::GemmProblem p{x + r * s->mod_kr * s->es, ldx, s->w_mod, s->mod_kr, (int)rows,
                             (int)s->mod_out, (int)s->mod_kr};
    return rowwise(p, partial, ldp, accumulate != 0, dt, st_);
  }
  const char* w_row = static_cast<const char*>(s->w_row);
  // attention part: input columns R_r, weight columns [0, Dr)
  if (layer == TP_ATTN_OUT || layer == TP_BLOCK_OUT) {
    const tpk::GemmProblem p{x + r * s->Dr * s->es, ldx, w_row, s->k_row, (int)rows, (int)s->D,
                             (int)s->Dr};
    if ((st = rowwise(p, partial, ldp, accumulate != 0, dt, st_)) != TP_OK) return st;
  }
  // MLP part: input columns (H*d if packed) + C_r, weight columns [Dr, Dr + Fr)
  if (layer == TP_MLP_DOWN || layer == TP_BLOCK_OUT) {
    const int64_t c0 = (layer == TP_BLOCK_OUT ? HD : 0) + r * s->Fr;
    const tpk::GemmProblem p{x + c0 * s->es, ldx, w_row + s->dn_col0 * s->es, s->k_row, (int)rows,
                             (int)s->D, (int)s->Fr};
    return rowwise(p, partial, ldp, layer == TP_BLOCK_OUT || accumulate != 0, dt, st_);
  }
  return TP_OK;
}

namespace {

constexpr int kMaxUlysses = 16;

// Shared checks of the two Ulysses re-layouts: degree, heads, dtype and the
// 16-byte granularity of one head block W = (heads / degree) * head_dim.
tp_status check_ulysses(int32_t degree, int32_t rank, int64_t n, int64_t heads, int64_t head_dim,
                        tp_dtype dt, size_t* es, int64_t* W) {
  if (degree < 1 || degree > kMaxUlysses)
    return fail(degree < 1 ? TP_ERR_ARG : TP_ERR_UNSUPPORTED, "degree %d not in [1, %d]", degree,
                kMaxUlysses);
  if (rank < 0 || rank >= degree) return fail(TP_ERR_ARG, "rank %d not in [0, %d)", rank, degree);
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_ARG, "unknown dtype");
  tp_status st = check_tokens(n);
  if (st != TP_OK) return st;
  if (n * degree > INT32_MAX) return fail(TP_ERR_UNSUPPORTED, "sequence longer than 2^31-1");
  if (heads < 1 || head_dim < 1) return fail(TP_ERR_ARG, "heads and head_dim must be positive");
  if (heads % degree)
    return fail(TP_ERR_DIVISIBILITY, "ulysses degree %d does not divide %lld heads", degree,
                (long long)heads);
  *es = dt == TP_BF16 ? 2 : 4;
  *W = heads / degree * head_dim;
  if ((*W * (int64_t)*es) % 16)
    return fail(TP_ERR_UNSUPPORTED, "a head block must be a multiple of 16 bytes");
  return TP_OK;
}

tp_status copy(const tpk::CopyBlocksArgs& a, hipStream_t stream) {
  const hipError_t e = tpk::launch_copy_blocks(a, stream);
  if (e != hipSuccess) return hip_fail(e, "re-layout launch");
  return TP_OK;
}

}  // namespace

TP_API tp_status tp_ulysses_seq_to_heads(const void* const* chunks, int32_t degree, int64_t ld_in,
                                         int64_t tokens_per_rank, int64_t heads, int64_t head_dim,
                                         int32_t blocks, int32_t rank, tp_dtype dtype, void* out,
                                         int64_t ldo, void* stream) {
  size_t es;
  int64_t W;
  tp_status st = check_ulysses(degree, rank, tokens_per_rank, heads, head_dim, dtype, &es, &W);
  if (st != TP_OK) return st;
  if (!chunks) return fail(TP_ERR_ARG, "chunks is NULL");
  if (blocks < 1 || blocks > 3) return fail(TP_ERR_ARG, "blocks (%d) not in [1, 3]", blocks);
  const int64_t HD = heads * head_dim, n = tokens_per_rank;
  for (int i = 0; i < degree; ++i)
    if ((st = check_matrix("chunks[i]", chunks[i], ld_in, blocks * HD, es)) != TP_OK) return st;
  if ((st = check_matrix("out", out, ldo, blocks * W, es)) != TP_OK) return st;
  if (n == 0) return TP_OK;
  const int64_t ob = span_bytes(n * degree, ldo, blocks * W, es);
  for (int i = 0; i < degree; ++i)
    if (overlap(out, ob, chunks[i], span_bytes(n, ld_in, blocks * HD, es)))
      return fail(TP_ERR_ARG, "out overlaps chunks[%d]", i);
  tpk::CopyBlocksArgs a{};
  a.rows = (int)n;
  a.chunks = (int)(W * (int64_t)es / 16);
  a.src_ld = ld_in * (int64_t)es;
  a.dst_ld = ldo * (int64_t)es;
  for (int sr = 0; sr < degree; ++sr)
    for (int b = 0; b < blocks; ++b) {
      a.src[a.n] = static_cast<const char*>(chunks[sr]) + (b * HD + rank * W) * (int64_t)es;
      a.dst[a.n] = static_cast<char*>(out) + (sr * n * ldo + b * W) * (int64_t)es;
      ++a.n;
    }
  return copy(a, static_cast<hipStream_t>(stream));
}

TP_API tp_status tp_ulysses_heads_to_seq(const void* const* parts, int32_t degree, int64_t ld_in,
                                         int64_t tokens_per_rank, int64_t heads, int64_t head_dim,
                                         int32_t rank, tp_dtype dtype, void* out, int64_t ldo,
                                         void* stream) {
  size_t es;
  int64_t W;
  tp_status st = check_ulysses(degree, rank, tokens_per_rank, heads, head_dim, dtype, &es, &W);
  if (st != TP_OK) return st;
  if (!parts) return fail(TP_ERR_ARG, "parts is NULL");
  const int64_t n = tokens_per_rank;
  for (int i = 0; i < degree; ++i)
    if ((st = check_matrix("parts[i]", parts[i], ld_in, W, es)) != TP_OK) return st;
  if ((st = check_matrix("out", out, ldo, heads * head_dim, es)) != TP_OK) return st;
  if (n == 0) return TP_OK;
  const int64_t ob = span_bytes(n, ldo, heads * head_dim, es);
  for (int i = 0; i < degree; ++i)
    if (overlap(out, ob, parts[i], span_bytes(n * degree, ld_in, W, es)))
      return fail(TP_ERR_ARG, "out overlaps parts[%d]", i);
  tpk::CopyBlocksArgs a{};
  a.rows = (int)n;
  a.chunks = (int)(W * (int64_t)es / 16);
  a.src_ld = ld_in * (int64_t)es;
  a.dst_ld = ldo * (int64_t)es;
  for (int r = 0; r < degree; ++r) {
    a.src[a.n] = static_cast<const char*>(parts[r]) + rank * n * ld_in * (int64_t)es;
    a.dst[a.n] = static_cast<char*>(out) + r * W * (int64_t)es;
    ++a.n;
  }
  return copy(a, static_cast<hipStream_t>(stream));
}

TP_API tp_status tp_partial_reduce(const float* const* partials, int32_t n_partials, int64_t ldp,
                                   const float* const* biases, int32_t n_biases, int64_t tokens,
                                   int64_t hidden, float* out, int64_t ldo, void* stream) {
  if (!partials) return fail(TP_ERR_ARG, "partials is NULL");
  if (n_partials < 1) return fail(TP_ERR_ARG, "n_partials (%d) < 1", n_partials);
  if (n_partials > tpk::kMaxReducePartials)
    return fail(TP_ERR_UNSUPPORTED, "n_partials (%d) > %d", n_partials, tpk::kMaxReducePartials);
  if (n_biases < 0) return fail(TP_ERR_ARG, "n_biases (%d) < 0", n_biases);
  if (n_biases > tpk::kMaxReduceBiases)
    return fail(TP_ERR_UNSUPPORTED, "n_biases (%d) > %d", n_biases, tpk::kMaxReduceBiases);
  if (n_biases > 0 && !biases) return fail(TP_ERR_ARG, "biases is NULL");
  tp_status st = check_tokens(tokens);
  if (st != TP_OK) return st;
  if (hidden <= 0 || hidden % 4) return fail(TP_ERR_ARG, "hidden (%lld) must be a positive multiple of 4",
                                            (long long)hidden);
  if (tokens * (hidden / 4) >= ((int64_t)1 << 31))
    return fail(TP_ERR_UNSUPPORTED, "tokens*hidden/4 >= 2^31");
  tpk::ReduceArgs a{};
  for (int i = 0; i < n_partials; ++i) {
    if ((st = check_matrix("partials[i]", partials[i], ldp, hidden, sizeof(float))) != TP_OK) return st;
    a.partials[i] = partials[i];
  }
  for (int i = 0; i < n_biases; ++i) {
    if (!biases[i]) return fail(TP_ERR_ARG, "biases[%d] is NULL", i);
    if (!aligned16(biases[i])) return fail(TP_ERR_ARG, "biases[%d] is not 16-byte aligned", i);
    a.biases[i] = biases[i];
  }
  if ((st = check_matrix("out", out, ldo, hidden, sizeof(float))) != TP_OK) return st;
  if (tokens == 0) return TP_OK;
  const int64_t ob = span_bytes(tokens, ldo, hidden, sizeof(float));
  for (int i = 0; i < n_partials; ++i) {
    const bool same = partials[i] == out && ldp == ldo;
    if (overlap(out, ob, partials[i], span_bytes(tokens, ldp, hidden, sizeof(float))) && !(i == 0 && same))
      return fail(TP_ERR_ARG, "out overlaps partials[%d] (only exact aliasing of partials[0] is allowed)", i);
  }
  for (int i = 0; i < n_biases; ++i)
    if (overlap(out, ob, biases[i], hidden * (int64_t)sizeof(float)))
      return fail(TP_ERR_ARG, "out overlaps biases[%d]", i);
  a.n_partials = n_partials;
  a.n_biases = n_biases;
  a.rows = tokens;
  a.cols = hidden;
  a.ldp = ldp;
  a.ldo = ldo;
  a.out = out;
  const hipError_t e = tpk::launch_partial_reduce(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reduce launch");
  return TP_OK;
}

TP_API const char* tp_status_string(tp_status status) {
  switch (status) {
    case TP_OK: return "TP_OK";
    case TP_ERR_ARG: return "TP_ERR_ARG: invalid argument";
    case TP_ERR_DIVISIBILITY: return "TP_ERR_DIVISIBILITY: tp_degree does not divide a sharded dimension";
    case TP_ERR_UNSUPPORTED: return "TP_ERR_UNSUPPORTED: combination not built";
    case TP_ERR_HIP: return "TP_ERR_HIP: HIP runtime error";
    case TP_ERR_OOM: return "TP_ERR_OOM: device allocation failed";
    case TP_ERR_IO: return "TP_ERR_IO: weight file missing, unreadable or too short";
  }
  return "unknown tp_status";
}

TP_API const char* tp_last_error_detail(void) { return g_detail.c_str(); }

}  // extern "C"
