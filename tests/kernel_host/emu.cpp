// Host runtime for the kernels compiled against tests/kernel_host/hip/hip_runtime.h,
// and a driver that runs the library's C entry points on host memory.
//
//   scan_host <mode> <dir>
//
// reads dir/args.txt ("name value" lines) and the input arrays dir/<name>.bin
// (raw little-endian, the dtype the entry point expects), calls the entry
// point with exact-size host buffers, and writes the outputs as
// dir/<name>.out.bin.  Modes: fwd (ss_scan_fwd_ex), noalloc
// (ss_scan_fwd_noalloc), bwd (ss_scan_bwd_ex), train (ss_scan_fwd_save then
// ss_scan_bwd_saved), step (ss_state_update_ex),
// cross (ss_cross_scan_fwd).  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer, so any access outside a tensor, outside the
// launch's LDS, or any undefined arithmetic ends the run with a report.
#include <hip/hip_runtime.h>

#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <fstream>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include <sanitizer/asan_interface.h>

#include "ss_scan.h"

namespace emu {

thread_local dim3 tl_thread, tl_block, tl_bdim, tl_gdim;
thread_local int tl_lane;

constexpr size_t kLdsMax = 160 * 1024;
alignas(256) static unsigned char g_lds[kLdsMax];
static size_t g_lds_bytes = 0;

// A barrier whose members may leave (a work-item that returns stops counting,
// as a finished wave stops counting at s_barrier); a wait that lasts longer
// than a minute aborts, so a protocol error ends the run instead of hanging it.
class Barrier {
public:
    void reset(int n) {
        std::lock_guard<std::mutex> g(m_);
        expected_ = n;
        count_ = 0;
    }
    void arrive_and_wait() {
        std::unique_lock<std::mutex> lk(m_);
        const long gen = gen_;
        if (++count_ >= expected_) {
            release();
            return;
        }
        if (!cv_.wait_for(lk, std::chrono::seconds(60), [&] { return gen_ != gen; })) {
            std::fprintf(stderr, "emu: barrier wait timed out (%d of %d arrived)\n", count_, expected_);
            std::abort();
        }
    }
    void drop() {
        std::lock_guard<std::mutex> g(m_);
        expected_--;
        if (expected_ > 0 && count_ >= expected_) release();
    }

private:
    void release() {
        count_ = 0;
        gen_++;
        cv_.notify_all();
    }
    std::mutex m_;
    std::condition_variable cv_;
    int expected_ = 0, count_ = 0;
    long gen_ = 0;
};

struct Wave {
    Barrier bar;
    uint32_t xa[64], xb[64];
};

static Barrier g_block_bar;
static std::vector<Wave*> g_waves;

static Wave& my_wave() { return *g_waves[tl_thread.x / 64]; }

void block_barrier() { g_block_bar.arrive_and_wait(); }
void wave_barrier() { my_wave().bar.arrive_and_wait(); }
void sleep_a_little() { std::this_thread::yield(); }
unsigned char* lds_base() { return g_lds; }

hipError_t get_device(int* dev) {
    *dev = 0;
    return hipSuccess;
}
static int g_cus = 4;   // a small machine, so that long scans are cut into segments
hipError_t device_attribute(int* v, int, int) {
    *v = g_cus;
    return hipSuccess;
}
hipError_t occupancy(int* nb, const void*, int, size_t) {
    *nb = 1;
    return hipSuccess;
}
hipError_t symbol_address(void** p, const void* sym) {
    *p = const_cast<void*>(sym);
    return hipSuccess;
}

// Work-item threads, kept across launches: thread t runs work-item t of
// every workgroup (the workgroups of a launch one after another).
class Pool {
public:
    void run(int nthreads, const std::function<void(int)>& item) {
        std::unique_lock<std::mutex> lk(m_);
        while (int(threads_.size()) < nthreads) {
            const int t = int(threads_.size());
            threads_.emplace_back([this, t] { worker(t); });
        }
        item_ = &item;
        active_ = nthreads;
        pending_ = nthreads;
        job_++;
        cv_.notify_all();
        done_cv_.wait(lk, [&] { return pending_ == 0; });
    }
    ~Pool() {
        {
            std::lock_guard<std::mutex> g(m_);
            stop_ = true;
            job_++;
        }
        cv_.notify_all();
        for (auto& t : threads_) t.join();
    }

private:
    void worker(int t) {
        long seen = 0;
        for (;;) {
            const std::function<void(int)>* item;
            {
                std::unique_lock<std::mutex> lk(m_);
                cv_.wait(lk, [&] { return job_ != seen; });
                seen = job_;
                if (stop_) return;
                if (t >= active_) continue;
                item = item_;
            }
            (*item)(t);
            std::lock_guard<std::mutex> g(m_);
            if (--pending_ == 0) done_cv_.notify_all();
        }
    }
    std::mutex m_;
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> threads_;
    const std::function<void(int)>* item_ = nullptr;
    int active_ = 0, pending_ = 0;
    long job_ = 0;
    bool stop_ = false;
};

void run_grid(dim3 grid, dim3 block, size_t lds, void (*body)(void*), void* ctx) {
    static Pool pool;
    if (lds > kLdsMax || block.y != 1 || block.z != 1 || grid.y != 1 || grid.z != 1 || block.x > 1024) {
        std::fprintf(stderr, "emu: launch shape not supported (lds %zu, block %u)\n", lds, block.x);
        std::abort();
    }
    // LDS past the launch's dynamic size is poisoned: touching it is an error.
    ASAN_UNPOISON_MEMORY_REGION(g_lds, kLdsMax);
    std::memset(g_lds, 0xA5, kLdsMax);
    ASAN_POISON_MEMORY_REGION(g_lds + lds, kLdsMax - lds);
    g_lds_bytes = lds;
    const int nthreads = int(block.x), nwaves = (nthreads + 63) / 64;
    for (unsigned bx = 0; bx < grid.x; bx++) {
        g_block_bar.reset(nthreads);
        for (auto* w : g_waves) delete w;
        g_waves.clear();
        for (int w = 0; w < nwaves; w++) {
            g_waves.push_back(new Wave());
            g_waves.back()->bar.reset(std::min(64, nthreads - 64 * w));
        }
        const std::function<void(int)> item = [&](int t) {
            tl_thread = dim3(unsigned(t), 0, 0);
            tl_block = dim3(bx, 0, 0);
            tl_bdim = block;
            tl_gdim = grid;
            tl_lane = t % 64;
            body(ctx);
            g_waves[t / 64]->bar.drop();
            g_block_bar.drop();
        };
        pool.run(nthreads, item);
    }
    ASAN_UNPOISON_MEMORY_REGION(g_lds, kLdsMax);
}

// Direct-to-LDS load: this lane's `bytes` land at lds_dst + lane * max(bytes, 4)
// (a 2-byte value is zero-extended into its 4-byte slot).
void global_load_lds(const void* src, void* lds_dst, int bytes) {
    unsigned char* dst = static_cast<unsigned char*>(lds_dst) + tl_lane * std::max(bytes, 4);
    if (dst < g_lds || dst + std::max(bytes, 4) > g_lds + g_lds_bytes) {
        std::fprintf(stderr, "emu: direct-to-LDS destination outside the launch's LDS\n");
        std::abort();
    }
    uint32_t w = 0;
    if (bytes < 4) {
        std::memcpy(&w, src, size_t(bytes));
        std::memcpy(dst, &w, 4);
    } else {
        std::memcpy(dst, src, size_t(bytes));
    }
}

// The same through a buffer descriptor.  The kernels size every descriptor
// to exactly the bytes they read, so an access past it is reported as an
// error here (the hardware would read zeros instead).
void buffer_load_lds(emu_rsrc r, uintptr_t lds_off, int bytes, uint32_t voff, uint32_t soff, uint32_t off) {
    const uint64_t at = uint64_t(soff) + voff + off;
    if (at + uint64_t(bytes) > r.bytes) {
        std::fprintf(stderr, "emu: buffer load at byte %llu of a %u-byte descriptor\n", (unsigned long long)at, r.bytes);
        std::abort();
    }
    global_load_lds(r.base + at, g_lds + lds_off, bytes);
}

// A buffer load into registers: `bytes` bytes at voff + soff, or 0 where they
// do not lie inside the descriptor's range (as the hardware's range check of
// an untyped buffer returns 0 for such lanes).
uint32_t buffer_load(emu_rsrc r, uint32_t voff, uint32_t soff, int bytes) {
    const uint64_t at = uint64_t(soff) + voff;
    if (at + uint64_t(bytes) > r.bytes) return 0u;
    uint32_t v = 0;
    std::memcpy(&v, r.base + at, size_t(bytes));
    return v;
}

// Cross-lane exchanges: every lane publishes, the wave meets, every lane
// reads what it needs, the wave meets again.
template <typename F>
static void exchange(uint32_t a, uint32_t b, F&& read) {
    Wave& w = my_wave();
    w.xa[tl_lane] = a;
    w.xb[tl_lane] = b;
    w.bar.arrive_and_wait();
    read(w);
    w.bar.arrive_and_wait();
}

// v_permlane32_swap: the upper 32 lanes of the first operand trade places
// with the lower 32 lanes of the second.
u32x2 permlane32_swap(unsigned a, unsigned b) {
    u32x2 r;
    exchange(a, b, [&](Wave& w) {
        const int l = tl_lane;
        r[0] = l < 32 ? w.xa[l] : w.xb[l - 32];
        r[1] = l < 32 ? w.xa[l + 32] : w.xb[l];
    });
    return r;
}

// v_permlane16_swap: the odd rows (of 16 lanes) of the first operand trade
// places with the even rows of the second.
u32x2 permlane16_swap(unsigned a, unsigned b) {
    u32x2 r;
    exchange(a, b, [&](Wave& w) {
        const int l = tl_lane;
        const bool odd = (l / 16) % 2 == 1;
        r[0] = odd ? w.xb[l - 16] : w.xa[l];
        r[1] = odd ? w.xb[l] : w.xa[l + 16];
    });
    return r;
}

// DPP with the controls the kernels use: quad_perm (0x00 .. 0xff: lane l of
// a quad reads quad position (ctrl >> 2 (l % 4)) & 3), row_shr:k (0x111 ..
// 0x11f: lane l takes lane l - k of its row of 16; lanes with no source take 0
// when bound_ctrl is set, else `old`) and row_ror:k (0x121 .. 0x12f: lane l
// takes lane (l - k) mod 16 of its row).
int update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl) {
    const bool quad = ctrl >= 0 && ctrl <= 0xff, shr = ctrl >= 0x111 && ctrl <= 0x11f,
               ror = ctrl >= 0x121 && ctrl <= 0x12f;
    if (!quad && !shr && !ror) {
        std::fprintf(stderr, "emu: DPP control 0x%x not emulated\n", ctrl);
        std::abort();
    }
    int res = old;
    exchange(uint32_t(src), 0, [&](Wave& w) {
        const int l = tl_lane, row = l / 16, bank = (l % 16) / 4;
        if (!((row_mask >> row) & 1) || !((bank_mask >> bank) & 1)) return;
        if (quad) {
            res = int(w.xa[(l & ~3) + ((ctrl >> (2 * (l % 4))) & 3)]);
        } else if (ror) {
            res = int(w.xa[row * 16 + (l % 16 + 16 - (ctrl - 0x120)) % 16]);
        } else {
            const int k = ctrl - 0x110;
            if (l % 16 >= k) res = int(w.xa[l - k]);
            else if (bound_ctrl) res = 0;
        }
    });
    return res;
}

// Lane (l & ~(width - 1)) + (src % width), as the hardware's ds_bpermute
// form of __shfl computes it.
float shfl(float v, int src, int width) {
    float r = v;
    exchange(__float_as_uint(v), 0, [&](Wave& w) {
        const int l = tl_lane;
        r = __uint_as_float(w.xa[(l & ~(width - 1)) + (src & (width - 1))]);
    });
    return r;
}

float shfl_xor(float v, int mask, int width) {
    float r = v;
    exchange(__float_as_uint(v), 0, [&](Wave& w) {
        const int l = tl_lane, src = l ^ mask;
        if ((src / width) == (l / width)) r = __uint_as_float(w.xa[src]);
    });
    return r;
}

}  // namespace emu

// ============================================================================ driver

namespace {

std::string g_dir;
std::map<std::string, long long> g_args;

long long arg(const char* k) {
    auto it = g_args.find(k);
    if (it == g_args.end()) {
        std::fprintf(stderr, "scan_host: missing argument %s\n", k);
        std::exit(2);
    }
    return it->second;
}

// An input array of exactly `bytes` bytes (null when the file is absent and
// the input is optional).
std::vector<void*> g_allocs;
void* load(const char* name, size_t bytes, bool optional = false) {
    const std::string path = g_dir + "/" + name + ".bin";
    std::ifstream f(path, std::ios::binary);
    if (!f) {
        if (optional) return nullptr;
        std::fprintf(stderr, "scan_host: missing input %s\n", path.c_str());
        std::exit(2);
    }
    void* p = std::malloc(bytes ? bytes : 1);
    f.read(static_cast<char*>(p), std::streamsize(bytes));
    if (size_t(f.gcount()) != bytes) {
        std::fprintf(stderr, "scan_host: %s holds %lld bytes, expected %zu\n", path.c_str(), (long long)f.gcount(), bytes);
        std::exit(2);
    }
    g_allocs.push_back(p);
    return p;
}
void* output(size_t bytes) {
    void* p = std::malloc(bytes ? bytes : 1);
    std::memset(p, 0xFF, bytes);   // NaN-filled: an element never written shows
    g_allocs.push_back(p);
    return p;
}
void save(const char* name, const void* p, size_t bytes) {
    std::ofstream f(g_dir + "/" + name + ".out.bin", std::ios::binary);
    f.write(static_cast<const char*>(p), std::streamsize(bytes));
}

int run(const std::string& mode) {
    const long long es = arg("dtype") == SS_BF16 ? 2 : 4;
    ss_set_test_plan(int(g_args.count("segments") ? arg("segments") : 0), int(g_args.count("waves") ? arg("waves") : 0),
                     0, 0, 0);
    if (mode == "fwd" || mode == "noalloc") {
        const long long b = arg("b"), L = arg("L"), d = arg("d_in"), n = arg("n");
        const size_t nel = size_t(b * L * d), nbc = size_t(b * L * n), nst = size_t(b * d * n);
        void* u = load("u", nel * es);
        void* dl = load("delta", nel * es);
        float* A = static_cast<float*>(load("A_log", size_t(d * n) * 4));
        void* B = load("B", nbc * es);
        void* C = load("C", nbc * es);
        float* D = static_cast<float*>(load("D", size_t(d) * 4));
        void* z = load("z", nel * es, true);
        float* bias = static_cast<float*>(load("delta_bias", size_t(d) * 4, true));
        float* h0 = static_cast<float*>(load("h0", nst * 4, true));
        void* y = output(nel * es);
        float* last = static_cast<float*>(output(nst * 4));
        int rc;
        if (mode == "fwd") {
            const size_t wsb = ss_scan_fwd_workspace_bytes(b, L, d, n, int(arg("dtype")));
            void* ws = std::aligned_alloc(256, (wsb + 255) / 256 * 256);
            rc = ss_scan_fwd_ex(u, dl, A, B, C, D, z, bias, int(arg("softplus")), h0, int(arg("zoh")), y, last, b, L, d,
                                n, int(arg("dtype")), ws, wsb, nullptr);
            std::free(ws);
        } else {
            rc = ss_scan_fwd_noalloc(u, dl, A, B, C, D, z, bias, int(arg("softplus")), h0, int(arg("zoh")), y, last, b,
                                     L, d, n, int(arg("dtype")), nullptr);
        }
        if (rc != SS_OK) return rc;
        save("y", y, nel * es);
        save("last_state", last, nst * 4);
        return 0;
    }
    if (mode == "bwd" || mode == "train") {
        // train: ss_scan_fwd_save, then ss_scan_bwd_saved from what it kept.
        const long long b = arg("b"), L = arg("L"), d = arg("d_in"), n = arg("n");
        const size_t nel = size_t(b * L * d), nbc = size_t(b * L * n), nst = size_t(b * d * n);
        void* u = load("u", nel * es);
        void* dl = load("delta", nel * es);
        float* A = static_cast<float*>(load("A_log", size_t(d * n) * 4));
        void* B = load("B", nbc * es);
        void* C = load("C", nbc * es);
        float* D = static_cast<float*>(load("D", size_t(d) * 4));
        void* z = load("z", nel * es, true);
        float* bias = static_cast<float*>(load("delta_bias", size_t(d) * 4, true));
        float* h0 = static_cast<float*>(load("h0", nst * 4, true));
        void* dy = load("dy", nel * es);
        float* dlast = static_cast<float*>(load("dlast", nst * 4, true));
        void* du = output(nel * es);
        void* ddl = output(nel * es);
        float* dA = static_cast<float*>(output(size_t(d * n) * 4));
        void* dB = output(nbc * es);
        void* dC = output(nbc * es);
        float* dD = static_cast<float*>(output(size_t(d) * 4));
        void* dz = z ? output(nel * es) : nullptr;
        float* dbias = bias ? static_cast<float*>(output(size_t(d) * 4)) : nullptr;
        float* dh0 = h0 ? static_cast<float*>(output(nst * 4)) : nullptr;
        int rc;
        if (mode == "bwd") {
            const size_t wsb = ss_scan_bwd_workspace_bytes(b, L, d, n, int(arg("dtype")));
            void* ws = std::aligned_alloc(256, (wsb + 255) / 256 * 256);
            rc = ss_scan_bwd_ex(u, dl, A, B, C, D, z, bias, int(arg("softplus")), h0, int(arg("zoh")), dy, dlast, du,
                                ddl, dA, dB, dC, dD, dz, dbias, dh0, b, L, d, n, int(arg("dtype")), ws, wsb, nullptr);
            std::free(ws);
        } else {
            const size_t ckb = ss_scan_checkpoint_bytes(b, L, d, n);
            float* ck = static_cast<float*>(output(std::max<size_t>(ckb, 4)));
            void* ypre = z ? output(nel * es) : nullptr;
            void* y = output(nel * es);
            float* last = static_cast<float*>(output(nst * 4));
            const size_t fwb = ss_scan_fwd_workspace_bytes(b, L, d, n, int(arg("dtype")));
            void* fws = std::aligned_alloc(256, (fwb + 255) / 256 * 256);
            rc = ss_scan_fwd_save(u, dl, A, B, C, D, z, bias, int(arg("softplus")), h0, int(arg("zoh")), y, last, ck,
                                  ypre, b, L, d, n, int(arg("dtype")), fws, fwb, nullptr);
            std::free(fws);
            if (rc != SS_OK) return rc;
            save("y", y, nel * es);
            save("last_state", last, nst * 4);
            save("checkpoints", ck, ckb);
            if (ypre) save("y_pre", ypre, nel * es);
            const size_t wsb = ss_scan_bwd_saved_workspace_bytes(b, L, d, n, int(arg("dtype")));
            void* ws = std::aligned_alloc(256, (wsb + 255) / 256 * 256);
            rc = ss_scan_bwd_saved(u, dl, A, B, C, D, z, bias, int(arg("softplus")), h0, int(arg("zoh")), ck, ypre,
                                   dy, dlast, du, ddl, dA, dB, dC, dD, dz, dbias, dh0, b, L, d, n,
                                   int(arg("dtype")), ws, wsb, nullptr);
            std::free(ws);
        }
        if (rc != SS_OK) return rc;
        save("du", du, nel * es);
        save("ddelta", ddl, nel * es);
        save("dA_log", dA, size_t(d * n) * 4);
        save("dB", dB, nbc * es);
        save("dC", dC, nbc * es);
        save("dD", dD, size_t(d) * 4);
        if (dz) save("dz", dz, nel * es);
        if (dbias) save("ddelta_bias", dbias, size_t(d) * 4);
        if (dh0) save("dinitial_state", dh0, nst * 4);
        return 0;
    }
    if (mode == "step") {
        const long long b = arg("b"), d = arg("d_in"), n = arg("n");
        const size_t nch = size_t(b * d), nst = size_t(b * d * n);
        float* state = static_cast<float*>(load("state", nst * 4));
        void* x = load("x", nch * es);
        void* dt = load("dt", nch * es);
        float* A = static_cast<float*>(load("A_log", size_t(d * n) * 4));
        void* B = load("B", size_t(b * n) * es);
        void* C = load("C", size_t(b * n) * es);
        float* D = static_cast<float*>(load("D", size_t(d) * 4));
        void* z = load("z", nch * es, true);
        float* bias = static_cast<float*>(load("dt_bias", size_t(d) * 4, true));
        void* y = output(nch * es);
        const int rc = ss_state_update_ex(state, x, dt, A, B, C, D, z, bias, int(arg("softplus")), int(arg("zoh")), y, b,
                                          d, n, int(arg("dtype")), nullptr);
        if (rc != SS_OK) return rc;
        save("y", y, nch * es);
        save("state", state, nst * 4);
        return 0;
    }
    if (mode == "cross") {
        const long long maps = arg("maps"), H = arg("H"), W = arg("W"), d = arg("d_in"), n = arg("n");
        const long long b = 4 * maps, L = H * W;
        void* x = load("x", size_t(maps * L * d) * es);
        void* dl = load("delta", size_t(b * L * d) * es);
        float* A = static_cast<float*>(load("A_log", size_t(4 * d * n) * 4));
        void* B = load("B", size_t(b * L * n) * es);
        void* C = load("C", size_t(b * L * n) * es);
        float* D = static_cast<float*>(load("D", size_t(4 * d) * 4));
        float* bias = static_cast<float*>(load("delta_bias", size_t(4 * d) * 4, true));
        float* y = static_cast<float*>(output(size_t(maps * L * d) * 4));
        float* last = static_cast<float*>(output(size_t(b * d * n) * 4));
        const int form = int(g_args.count("form") ? arg("form") : SS_CROSS_AUTO);
        const size_t wsb = ss_cross_scan_fwd_ex_workspace_bytes(maps, H, W, d, n, int(arg("dtype")), form);
        void* ws = std::aligned_alloc(256, (wsb + 255) / 256 * 256);
        const int rc = ss_cross_scan_fwd_ex(x, dl, A, B, C, D, bias, int(arg("softplus")), y, last, maps, H, W, d, n,
                                            int(arg("dtype")), form, ws, wsb, nullptr);
        std::free(ws);
        if (rc != SS_OK) return rc;
        save("y", y, size_t(maps * L * d) * 4);
        save("last_state", last, size_t(b * d * n) * 4);
        return 0;
    }
    std::fprintf(stderr, "scan_host: unknown mode %s\n", mode.c_str());
    return 2;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: scan_host <fwd|noalloc|bwd|train|step|cross> <dir>\n");
        return 2;
    }
    g_dir = argv[2];
    std::ifstream f(g_dir + "/args.txt");
    std::string k;
    long long v;
    while (f >> k >> v) g_args[k] = v;
    if (g_args.count("cus")) emu::g_cus = int(g_args["cus"]);
    const int rc = run(argv[1]);
    for (void* p : g_allocs) std::free(p);
    if (rc != 0) std::fprintf(stderr, "scan_host: status %d (%s)\n", rc, ss_status_string(rc));
    return rc == 0 ? 0 : 1;
}
