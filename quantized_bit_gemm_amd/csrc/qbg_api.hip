// qbg_api.hip -- the C ABI (include/qbg.h): argument validation, the per-shape
// configuration table and its lookup, workspace sizing, and dispatch to the
// kernel launchers.
//
// Every entry point validates all arguments before making any HIP call, so a
// bad call returns its status code without touching the device.  The
// configuration table follows the pages' precomputed per-shape configs with a
// default for shapes outside the table ("Helion nel backend vLLM", ai-radar.it,
// paragraphs 3, 4 and 7): entries are keyed by (op, next power of two >= M,
// N, K) and carry the algorithmic variant (swap_ab, split_k) and the tile
// variant (kernel_id).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cerrno>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <dlfcn.h>
#include <fstream>
#include <memory>
#include <mutex>
#include <sstream>
#include <string>
#include <unordered_map>

#include "../../include/qbg.h"
#include "qbg_launch.h"

// Scratch of qbg_scaled_mm_noalloc: the slot region (64 KiB of split-K arrival
// counters, zero between calls) followed by room for the split-K partials.
// Each GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory: host
// code uses only the per-device address that device_scratch() takes once.
static __device__ __align__(256) unsigned char scratch[QBG_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

qbg_status fail(qbg_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

qbg_status ok() {
    g_last_error.clear();
    return QBG_OK;
}

bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("QBG_LOG");
        return v && v[0] && v[0] != '0';
    }();
    return on;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

qbg_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(QBG_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Sizes the kernels index with 32-bit integers stay below this bound.
constexpr int64_t kMaxDim = (int64_t)1 << 30;
// Tokens of one GEMM call: decode (up to 32) through prefill batches.
constexpr int64_t kMaxTokens = 8192;
// Rows of one quantizer call (one workgroup per row; the grid's thread count
// stays below 2^32 at 1024 threads per row).
constexpr int64_t kMaxRows = (int64_t)1 << 22;
// 1 x 128 groups of one group-quantizer call (16 threads per group).
constexpr int64_t kMaxGroups = (int64_t)1 << 27;
// Weight bytes of one GEMM: the register-streaming kernel addresses a lane's
// weight row with a 32-bit offset.
constexpr int64_t kMaxWeightBytes = (int64_t)1 << 32;

// ---- configuration table --------------------------------------------------

struct Key {
    int op;
    int64_t mb, n, k;
    bool operator==(const Key& o) const { return op == o.op && mb == o.mb && n == o.n && k == o.k; }
};
struct KeyHash {
    size_t operator()(const Key& k) const {
        size_t h = (size_t)k.op * 1000003u;
        h ^= (size_t)k.mb + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
        h ^= (size_t)k.n + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
        h ^= (size_t)k.k + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
        return h;
    }
};
struct Entry {
    int kernel_id, swap_ab, split_k, rotate, fuse;
};
using Table = std::unordered_map<Key, Entry, KeyHash>;
std::shared_ptr<const Table> g_table;
// Set once any table has been installed (an explicit qbg_config_table_load or the
// automatic load below); the automatic load then does nothing.
std::atomic<bool> g_table_installed{false};
std::once_flag g_autoload_once;
qbg_status load_table_file(const char* path);

// The table a caller gets without loading one: the file QBG_CONFIG_TABLE names
// (set but empty: none, the built-in defaults only), else configs/gfx950.txt
// beside the loaded libqbg.so -- the tuned table shipped with the library
// ("Helion nel backend vLLM", ai-radar.it, paragraph 7: a default configuration
// for tests and CI, tuned configurations for deployment).  Loaded once, before
// the first lookup reads the table; a file that is missing or malformed leaves
// the built-in defaults (QBG_LOG=1 reports why).
void autoload_table() {
    std::call_once(g_autoload_once, [] {
        if (g_table_installed.load()) return;
        std::string path;
        if (const char* env = std::getenv("QBG_CONFIG_TABLE")) {
            path = env;
        } else {
            Dl_info info{};
            if (dladdr(reinterpret_cast<void*>(&autoload_table), &info) && info.dli_fname) {
                const std::string so = info.dli_fname;
                const size_t slash = so.rfind('/');
                path = (slash == std::string::npos ? std::string() : so.substr(0, slash + 1)) +
                       "configs/gfx950.txt";
            }
        }
        if (path.empty()) return;
        const std::string saved = g_last_error;  // the caller's last error stays as it was
        const qbg_status st = load_table_file(path.c_str());
        if (st != QBG_OK && log_enabled())
            std::fprintf(stderr, "[qbg] no tuned table loaded (%s): %s\n", path.c_str(),
                         g_last_error.c_str());
        g_last_error = saved;
    });
}

// Lookup flags from the environment, read once on the first lookup:
//   QBG_MAX_TUNED_M=n        table entries serve token counts up to n; a larger M
//                            gets the built-in default (unset: every bucket);
//   QBG_FORCE_CONFIG=k,s,p[,r[,f]]  every lookup returns kernel_id k, swap_ab s,
//                            split_k p, rotate r, fuse f (a debugging override;
//                            a call it does not fit fails with QBG_E_CONFIG).
// A malformed value is ignored (and reported with QBG_LOG).
struct LookupFlags {
    int64_t max_tuned_m = 0;
    bool force = false;
    Entry forced{0, 0, 1, 0, 0};
};

const LookupFlags& lookup_flags() {
    static const LookupFlags flags = [] {
        LookupFlags f;
        if (const char* v = std::getenv("QBG_MAX_TUNED_M")) {
            char* end = nullptr;
            const long long m = std::strtoll(v, &end, 10);
            if (end != v && *end == '\0' && m >= 1)
                f.max_tuned_m = m;
            else if (log_enabled())
                std::fprintf(stderr, "[qbg] ignoring QBG_MAX_TUNED_M=%s\n", v);
        }
        if (const char* v = std::getenv("QBG_FORCE_CONFIG")) {
            int x[5] = {0, 0, 1, 0, 0};
            int n = 0;
            const char* q = v;
            while (n < 5) {
                char* end = nullptr;
                const long val = std::strtol(q, &end, 10);
                if (end == q || val < 0 || val > 1000000) break;
                x[n++] = (int)val;
                q = end;
                if (*q != ',') break;
                ++q;
            }
            if (n >= 3 && *q == '\0') {
                f.force = true;
                f.forced = Entry{x[0], x[1], x[2], x[3], x[4]};
            } else if (log_enabled()) {
                std::fprintf(stderr, "[qbg] ignoring QBG_FORCE_CONFIG=%s\n", v);
            }
        }
        return f;
    }();
    return flags;
}

int64_t next_pow2(int64_t m) {
    int64_t b = 1;
    while (b < m) b <<= 1;
    return b;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int op_from_name(const std::string& s) {
    if (s == "fp8") return QBG_OP_FP8;
    if (s == "int8") return QBG_OP_INT8;
    if (s == "block_fp8") return QBG_OP_BLOCK_FP8;
    if (s == "block_ue8m0") return QBG_OP_BLOCK_UE8M0;
    if (s == "fp8_fused") return QBG_OP_FP8_FUSED;
    if (s == "int8_fused") return QBG_OP_INT8_FUSED;
    if (s == "fp8_grouped") return QBG_OP_FP8_GROUPED;
    if (s == "int8_grouped") return QBG_OP_INT8_GROUPED;
    return -1;
}

bool is_block(int op) { return op == QBG_OP_BLOCK_FP8 || op == QBG_OP_BLOCK_UE8M0; }
bool is_fused(int op) { return op == QBG_OP_FP8_FUSED || op == QBG_OP_INT8_FUSED; }
bool is_grouped(int op) { return op == QBG_OP_FP8_GROUPED || op == QBG_OP_INT8_GROUPED; }
bool op_valid(int op) { return op >= QBG_OP_FP8 && op <= QBG_OP_INT8_GROUPED; }

// An enum argument comes from C, where any int value can be passed, and
// reading an out-of-range value through a C++ enum type is undefined: entry
// points read the argument's bytes as an int and validate that.
template <class E>
int raw_enum(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "the C enums are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

// The kernel-level op a configuration runs: the fused ops resolve by their
// fuse mode to the producer launch, the LOCAL launch, or (SEPARATE) the plain
// op after a standalone quantizer launch.
int kernel_op(int op, int fuse) {
    if (!is_fused(op)) return op;
    const bool fp8 = op == QBG_OP_FP8_FUSED;
    if (fuse == QBG_FUSE_LOCAL) return fp8 ? qbg::OP_FP8_LOCAL : qbg::OP_INT8_LOCAL;
    if (fuse == QBG_FUSE_SEPARATE) return fp8 ? QBG_OP_FP8 : QBG_OP_INT8;
    return op;
}

// Routed rows a grouped call may carry.
constexpr int64_t kMaxGroupedRows = 65536;
constexpr int64_t kMaxExperts = 65535;
// Experts of a grouped call on the prefill tiles: every wave of those tiles
// scans the offsets, 64 experts at a time.
constexpr int64_t kMaxPrefillExperts = 1024;

// Poll iterations of the fused launch's bounded wait (qbg_set_fused_wait_limit).
std::atomic<int> g_wait_limit{qbg::kDefaultWaitLimit};

// Granularity of one split-K chunk: 16 bytes per lane load, one 128 group for blocks.
int64_t chunk_quantum(int op) { return is_block(op) ? 128 : 16; }

// Built-in configuration for shapes the table does not cover: enough
// workgroups to cover the 256 CUs several times, preferring no split.
// Above 32 tokens the per-channel ops take the large-M tile of 32 weight rows
// x 256 tokens, every token in one launch.
int large_m_default_kernel() {
    for (int k = 0; k < qbg::gemm_kernel_count(); ++k) {
        const qbg::TileShape t = qbg::gemm_tile(k);
        if (t.tm == 256 && qbg::tile_n(t) == 32) return k;
    }
    return -1;
}

// The prefill tile the default picks for the per-channel ops from 1024 tokens on: 128 weight
// rows x 256 tokens per workgroup (many workgroups at mid sizes, near the
// best tile at large ones).
int prefill_default_kernel() {
    for (int k = 0; k < qbg::gemm_kernel_count(); ++k) {
        const qbg::TileShape t = qbg::gemm_tile(k);
        if (t.big > 0 && t.tm == 256 && qbg::tile_n(t) == 128) return k;
    }
    return -1;
}

// Output tiles of a prefill-tile launch (one launch covers every token).
int64_t prefill_tiles(int64_t M, int64_t N, const qbg::TileShape& t) {
    return (M + t.tm - 1) / t.tm * ((N + qbg::tile_n(t) - 1) / qbg::tile_n(t));
}

Entry default_config(int op, int64_t M, int64_t N, int64_t K) {
    // Per-channel ops from 1024 tokens: the prefill tile (K a multiple of its
    // stage); past one decode launch otherwise: the large-M tile.  Otherwise 32 weight rows per
    // workgroup, 4 waves along K (the fused ops: the standalone quantizer,
    // then that GEMM); the grouped launch needs an
    // LDS-staged variant: 16 rows, 512-byte stage rows, 3 stages, Swap-AB.
    if (is_grouped(op)) return Entry{16, 1, 1, 0, 0};  // one launch per expert row group; no split
    const int fuse = is_fused(op) ? QBG_FUSE_SEPARATE : 0;
    const bool per_channel = op == QBG_OP_FP8 || op == QBG_OP_INT8 || is_fused(op);
    const int pk = prefill_default_kernel();
    if (per_channel && M >= 1024 && pk >= 0 && K % qbg::gemm_tile(pk).kb == 0) {
        // fewer output tiles than CUs and a long K loop: two K chunks per tile
        const bool split = prefill_tiles(M, N, qbg::gemm_tile(pk)) < 256 && K >= 8192 && K % 256 == 0;
        return Entry{pk, 0, split ? 2 : 1, 0, fuse};
    }
    // Block-FP8 from 1024 tokens: the 128 x 128 prefill tile (UE8M0: its codes fit
    // in LDS for the longest K)
    if (is_block(op) && M >= 1024 && (op != QBG_OP_BLOCK_UE8M0 || K % 512 == 0)) {
        for (int k = 0; k < qbg::gemm_kernel_count(); ++k) {
            const qbg::TileShape t = qbg::gemm_tile(k);
            if (t.big > 0 && t.tm == 128 && qbg::tile_n(t) == 128 &&
                qbg::gemm_lds_bytes(k, op, (int)M, K, K) <= qbg::kMaxLdsPerWorkgroup)
                return Entry{k, 0, 1, 0, 0};
        }
    }
    if (per_channel && M > qbg::kMaxTokensPerLaunch && large_m_default_kernel() >= 0)
        return Entry{large_m_default_kernel(), 1, 1, 0, fuse};
    Entry e{4, 0, 1, 0, fuse};
    const qbg::TileShape t = qbg::gemm_tile(e.kernel_id);
    const int64_t tiles = (N + qbg::tile_n(t) - 1) / qbg::tile_n(t);
    int64_t s = 1;
    while (tiles * s < 512 && s < 256 && (K % (2 * s)) == 0 &&
           ((K / (2 * s)) % chunk_quantum(op)) == 0 && (K / (2 * s)) >= 512)
        s *= 2;
    e.split_k = (int)s;
    return e;
}

qbg_status check_config(int op, int64_t K, const qbg_gemm_config& c) {
    if (c.kernel_id < 0 || c.kernel_id >= qbg::gemm_kernel_count())
        return fail(QBG_E_CONFIG, "kernel_id " + std::to_string(c.kernel_id) + " out of range");
    if (c.swap_ab != 0 && c.swap_ab != 1) return fail(QBG_E_CONFIG, "swap_ab must be 0 or 1");
    if (c.rotate != 0 && c.rotate != 1) return fail(QBG_E_CONFIG, "rotate must be 0 or 1");
    if (is_fused(op) ? (c.fuse < QBG_FUSE_PUBLISH || c.fuse > QBG_FUSE_SEPARATE) : c.fuse != 0)
        return fail(QBG_E_CONFIG, is_fused(op) ? "fuse must be a qbg_fuse_mode"
                                               : "fuse applies to the fused ops only");
    if (is_fused(op) && c.fuse == QBG_FUSE_LOCAL && qbg::gemm_tile(c.kernel_id).tm > 0)
        return fail(QBG_E_CONFIG, "LOCAL fusion runs on the decode tiles (tile_m 32)");
    if (is_fused(op) && c.fuse == QBG_FUSE_LOCAL && qbg::gemm_tile(c.kernel_id).ns == 0) {
        const qbg::TileShape t = qbg::gemm_tile(c.kernel_id);
        const int64_t two_groups = 2 * 128 * (int64_t)t.wk * t.ku;
        if (c.split_k < 1 || K % c.split_k != 0 || K / c.split_k != two_groups)
            return fail(QBG_E_CONFIG, "LOCAL on a register tile (stages 0): K / split_k must be "
                                      "two load groups of every wave, " + std::to_string(two_groups) +
                                      " bytes for kernel_id " + std::to_string(c.kernel_id));
    }
    if (qbg::gemm_tile(c.kernel_id).big > 0 && (c.swap_ab != 0 || K % qbg::gemm_tile(c.kernel_id).kb != 0))
        return fail(QBG_E_CONFIG, "prefill tiles run the Standard layout, K a multiple of " +
                                      std::to_string(qbg::gemm_tile(c.kernel_id).kb));
    if (qbg::gemm_tile(c.kernel_id).big > 0 && c.split_k != 1) {
        // split-K on the prefill tiles: the plain GEMMs, whole 128-byte stages (one
        // scale group each) per chunk
        const int kop = kernel_op(op, c.fuse);
        if (kop != QBG_OP_FP8 && kop != QBG_OP_INT8 && !is_block(kop))
            return fail(QBG_E_CONFIG, "prefill tiles split K for the plain FP8, INT8 and Block-FP8 GEMMs only");
        if (c.split_k > 16 || K % ((int64_t)c.split_k * 128) != 0)
            return fail(QBG_E_CONFIG, "prefill tiles split K in at most 16 chunks of a multiple of 128");
    }
    if (qbg::gemm_tile(c.kernel_id).big > 0 && op == QBG_OP_BLOCK_UE8M0 && K % 512 != 0)
        return fail(QBG_E_CONFIG, "prefill tiles run Block-FP8 with K a multiple of 512");
    if (!qbg::gemm_kernel_supports(c.kernel_id, kernel_op(op, c.fuse)))
        return fail(QBG_E_CONFIG, "kernel_id " + std::to_string(c.kernel_id) +
                                      " does not support this op");
    if (!is_pow2(c.split_k) || c.split_k > 256)
        return fail(QBG_E_SPLITK, "split_k must be a power of two <= 256");
    if (is_grouped(op) && c.split_k != 1)
        return fail(QBG_E_SPLITK, "the grouped GEMM runs without split-K");
    if (K % c.split_k != 0 || (K / c.split_k) % chunk_quantum(op) != 0)
        return fail(QBG_E_SPLITK, "K / split_k must be a multiple of " +
                                      std::to_string(chunk_quantum(op)));
    return QBG_OK;
}

qbg_status check_lds(int op, int64_t M, int64_t K, const qbg_gemm_config& c) {
    if (qbg::gemm_lds_bytes(c.kernel_id, kernel_op(op, c.fuse), (int)M, K, K / c.split_k) >
        qbg::kMaxLdsPerWorkgroup)
        return fail(QBG_E_CONFIG, "kernel_id " + std::to_string(c.kernel_id) +
                                      " needs more LDS than a CU has at M=" + std::to_string(M) +
                                      ", K chunk " + std::to_string(K / c.split_k));
    return QBG_OK;
}

void fill_tile(qbg_gemm_config* c) {
    const qbg::TileShape t = qbg::gemm_tile(c->kernel_id);
    c->tile_n = qbg::tile_n(t);
    c->waves_n = t.wn;
    c->waves_k = t.wk;
    c->k_unroll = t.ku;
    c->stages = t.ns;
    c->waves_m = t.wm;
    c->tile_m = qbg::tile_tokens(t);
}

qbg_gemm_config resolve(int op, int64_t M, int64_t N, int64_t K, const qbg_gemm_config* cfg,
                        int* from_table) {
    qbg_gemm_config c{};
    if (from_table) *from_table = 0;
    if (cfg) {
        c.kernel_id = cfg->kernel_id;
        c.swap_ab = cfg->swap_ab;
        c.split_k = cfg->split_k;
        c.rotate = cfg->rotate;
        c.fuse = cfg->fuse;
    } else {
        autoload_table();
        const LookupFlags& flags = lookup_flags();
        std::shared_ptr<const Table> t = std::atomic_load(&g_table);
        Entry e;
        bool hit = false;
        if (flags.force) {
            e = flags.forced;
        } else {
            if (t && (flags.max_tuned_m == 0 || M <= flags.max_tuned_m)) {
                auto it = t->find(Key{op, next_pow2(M), N, K});
                if (it != t->end()) {
                    e = it->second;
                    hit = true;
                }
            }
            if (!hit) e = default_config(op, M, N, K);
        }
        if (from_table) *from_table = hit ? 1 : 0;
        c.kernel_id = e.kernel_id;
        c.swap_ab = e.swap_ab;
        c.split_k = e.split_k;
        c.rotate = e.rotate;
        c.fuse = e.fuse;
    }
    if (c.kernel_id >= 0 && c.kernel_id < qbg::gemm_kernel_count()) fill_tile(&c);
    return c;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace layout, the same for every shape: a fixed 64 KiB region of 32-bit
// slots (the fused launch's synchronization slots, then one split-K arrival
// counter per output tile; all zero between calls), then the partials of one
// launch (at most the tile's tokens per launch).  Because the slots never share
// bytes with any shape's partials, one zero-initialized workspace serves calls
// of every shape and configuration.
constexpr int64_t kSlotCount = 16384;
constexpr size_t kCounterBytes = (size_t)kSlotCount * 4;
constexpr int64_t kCounterSlots = kSlotCount - qbg::kSyncSlots;  // split-K tiles

int64_t tiles_of(int64_t N, const qbg_gemm_config& c) {
    const int64_t tn = c.tile_n > 0 ? c.tile_n : 16;
    return (N + tn - 1) / tn;
}

size_t workspace_bytes(int op, int64_t M, int64_t N, const qbg_gemm_config& c) {
    const bool slots = is_fused(op) && c.fuse == QBG_FUSE_PUBLISH;
    if (c.split_k <= 1) return slots ? kCounterBytes : 0;
    const qbg::TileShape t = qbg::gemm_tile(c.kernel_id);
    if (t.big > 0)  // each chunk's whole tiles, 4-byte sums
        return kCounterBytes +
               align256((size_t)prefill_tiles(M, N, t) * c.split_k * t.tm * qbg::tile_n(t) * 4);
    const int64_t cap = qbg::tile_tokens(qbg::gemm_tile(c.kernel_id));
    const int64_t m = M < cap ? M : cap;
    return kCounterBytes + align256((size_t)c.split_k * m * N * 4);
}

qbg_status check_gemm_shape(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kMaxTokens) return fail(QBG_E_SHAPE, "M must be in [1, 8192]");
    if (N < 16 || N % 16 != 0 || N > kMaxDim) return fail(QBG_E_SHAPE, "N must be a positive multiple of 16");
    if (K < 16 || K % 16 != 0 || K > kMaxDim) return fail(QBG_E_SHAPE, "K must be a positive multiple of 16");
    if (N * K >= kMaxWeightBytes) return fail(QBG_E_SHAPE, "N * K must be below 2^32 bytes");
    return QBG_OK;
}

static_assert(QBG_NOALLOC_SCRATCH_BYTES % 256 == 0 && QBG_NOALLOC_SCRATCH_BYTES > kCounterBytes,
              "the scratch holds the slot region and some partials");
constexpr int kMaxScratchDevices = 64;

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxScratchDevices];

// Device address of this GPU's `scratch` for a launch on `stream`, which must
// belong to the current device.  The first call on a device takes the address
// (hipGetSymbolAddress, with that device current) and clears the slot region
// with the fill kernel on `stream`, ahead of the caller's launches; device
// globals also start zeroed when the code object loads.  Every later call
// finds the slots zero again, because each split-K launch's last arrival
// resets its counter.
qbg_status device_scratch(void* stream, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(QBG_E_SHAPE, "qbg_scaled_mm_noalloc supports device indexes below 64");
    if (stream) {
        int sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
        if (sdev != dev) return fail(QBG_E_SHAPE, "the stream belongs to another device than the current one");
    }
    DeviceScratch& d = g_scratch[dev];
    std::call_once(d.once, [&] {
        d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess)
            d.err = qbg::launch_fill_zero(d.ptr, kCounterBytes, static_cast<hipStream_t>(stream));
        if (d.err != hipSuccess) d.ptr = nullptr;
    });
    if (d.err != hipSuccess || !d.ptr) return hip_status(d.err != hipSuccess ? d.err : hipErrorUnknown,
                                                          "scratch set-up");
    *out = d.ptr;
    return QBG_OK;
}

// Shared GEMM driver: resolve the configuration, validate the workspace and
// enqueue one launch per slice of at most the tile's tokens per launch.  For the
// fused ops `x` holds the bf16 activations and a_q / a_scale receive their
// quantization (each slice's launch quantizes its own rows).  With
// static_scratch the launches use this GPU's `scratch` instead of `workspace`.
qbg_status run_gemm(int op, const void* a_q, const void* a_scale, const void* w_q,
                    const void* w_scale, int64_t M, int64_t N, int64_t K, void* out, int raw_i32,
                    const qbg_gemm_config* cfg, void* workspace, size_t ws_bytes, void* stream,
                    const void* x = nullptr, bool static_scratch = false) {
    if (!a_q || !w_q || !out || (!raw_i32 && (!a_scale || !w_scale)) || (is_fused(op) && !x))
        return fail(QBG_E_NULL, "null tensor pointer");
    qbg_status st = check_gemm_shape(M, N, K);
    if (st != QBG_OK) return st;
    if (is_fused(op) && !aligned(x, 16)) return fail(QBG_E_ALIGN, "x must be 16-byte aligned");
    if (is_block(op) && K % 128 != 0) return fail(QBG_E_SHAPE, "block GEMM needs K % 128 == 0");
    if (!aligned(a_q, 16) || !aligned(w_q, 16)) return fail(QBG_E_ALIGN, "operands must be 16-byte aligned");
    const size_t scale_align = op == QBG_OP_BLOCK_UE8M0 ? 1 : 4;
    if (!aligned(out, 4) || (a_scale && !aligned(a_scale, scale_align)) ||
        (w_scale && !aligned(w_scale, scale_align)))
        return fail(QBG_E_ALIGN, "outputs and fp32 scales must be 4-byte aligned");
    int from_table = 0;
    const qbg_gemm_config c = resolve(op, M, N, K, cfg, &from_table);
    st = check_config(op, K, c);
    if (st != QBG_OK) return st;
    st = check_lds(op, M, K, c);
    if (st != QBG_OK) return st;
    if (qbg::gemm_tile(c.kernel_id).big > 0 && op == QBG_OP_BLOCK_UE8M0 &&
        (!aligned(a_scale, 4) || !aligned(w_scale, 4)))
        return fail(QBG_E_ALIGN, "the prefill tiles read UE8M0 scale codes as 4-byte words: "
                                 "a_scale and w_scale must be 4-byte aligned");
    const size_t need = workspace_bytes(op, M, N, c);
    const qbg::TileShape tile = qbg::gemm_tile(c.kernel_id);
    if (c.split_k > 1 && (tile.big > 0 ? prefill_tiles(M, N, tile) : tiles_of(N, c)) > kCounterSlots)
        return fail(QBG_E_SHAPE, "split_k > 1 supports at most " + std::to_string(kCounterSlots) +
                                     " output tiles");
    if (static_scratch) {
        if (need > QBG_NOALLOC_SCRATCH_BYTES)
            return fail(QBG_E_WORKSPACE,
                        "this call needs " + std::to_string(need) + " bytes of scratch, more than the " +
                            std::to_string((size_t)QBG_NOALLOC_SCRATCH_BYTES) +
                            " that qbg_scaled_mm_noalloc holds: force a configuration with a smaller "
                            "split_k, or call qbg_scaled_mm with a workspace");
        if (need > 0) {
            st = device_scratch(stream, &workspace);
            if (st != QBG_OK) return st;
            ws_bytes = QBG_NOALLOC_SCRATCH_BYTES;
        }
    }
    if (need > 0) {
        if (!workspace)
            return fail(QBG_E_WORKSPACE, c.split_k <= 1 ? "the fused launch needs a workspace"
                                                        : "split_k > 1 needs a workspace");
        if (ws_bytes < need)
            return fail(QBG_E_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
        if (!aligned(workspace, 256)) return fail(QBG_E_ALIGN, "workspace must be 256-byte aligned");
    }
    if (log_enabled())
        std::fprintf(stderr, "[qbg] op=%d M=%lld N=%lld K=%lld kernel=%d swap_ab=%d split_k=%d rotate=%d fuse=%d tile_n=%d%s\n",
                     op, (long long)M, (long long)N, (long long)K, c.kernel_id, c.swap_ab, c.split_k,
                     c.rotate, c.fuse, c.tile_n, cfg ? " (forced)" : (from_table ? " (table)" : " (default)"));

    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int kop = kernel_op(op, c.fuse);
    // A large-M tile without split-K, and a prefill tile, cover every token in
    // one launch; otherwise the tokens run as launches of at most the tile's tokens.
    const bool one_launch = tile.tm > 0 && (c.split_k == 1 || tile.big > 0);
    if (is_fused(op) && c.fuse == QBG_FUSE_SEPARATE) {
        // two launches: the standalone quantizer writes a_q / a_scale, the GEMM reads them
        hipError_t e = qbg::launch_quant_per_token(op == QBG_OP_FP8_FUSED ? 0 : 1, x, M, K,
                                                   const_cast<void*>(a_q),
                                                   static_cast<float*>(const_cast<void*>(a_scale)), s);
        if (e != hipSuccess) return hip_status(e, "quantizer launch");
    }
    const int64_t kg = K / 128;
    const int64_t cap = one_launch ? M : qbg::tile_tokens(tile);
    for (int64_t m0 = 0; m0 < M; m0 += cap) {
        const int64_t mm = (M - m0) < cap ? (M - m0) : cap;
        qbg::GemmArgs p{};
        p.a = static_cast<const uint8_t*>(a_q) + m0 * K;
        p.w = static_cast<const uint8_t*>(w_q);
        p.w_scale = w_scale;
        if (is_block(op)) {
            const size_t esz = op == QBG_OP_BLOCK_UE8M0 ? 1 : 4;
            p.a_scale = static_cast<const char*>(a_scale) + (size_t)(m0 * kg) * esz;
        } else {
            p.a_scale = a_scale ? static_cast<const float*>(a_scale) + m0 : nullptr;
        }
        p.out = static_cast<char*>(out) + (size_t)(m0 * N) * (raw_i32 ? 4 : 2);
        p.sync = need > 0 ? static_cast<uint32_t*>(workspace) : nullptr;
        p.counters = need > 0 ? static_cast<uint32_t*>(workspace) + qbg::kSyncSlots : nullptr;
        p.partial = c.split_k > 1 ? static_cast<char*>(workspace) + kCounterBytes : nullptr;
        p.x = x ? static_cast<const uint16_t*>(x) + m0 * K : nullptr;
        if (qbg::op_is_local(kop)) {
            p.a_out = static_cast<uint8_t*>(const_cast<void*>(a_q)) + m0 * K;
            p.a_scale_out = static_cast<float*>(const_cast<void*>(a_scale)) + m0;
        }
        p.wait_limit = g_wait_limit.load(std::memory_order_relaxed);
        p.M = (int)mm;
        p.N = (int)N;
        p.K = (int)K;
        p.split_k = c.split_k;
        p.k_chunk = (int)(K / c.split_k);
        p.raw_i32 = raw_i32;
        p.kgroups = (int)kg;
        p.rotate = c.rotate;
        hipError_t e = qbg::launch_gemm(kop, p, c.kernel_id, c.swap_ab, s);
        if (e != hipSuccess) return hip_status(e, "GEMM launch");
    }
    return ok();
}

qbg_status load_table_file(const char* path) {
    if (!path) return fail(QBG_E_NULL, "null path");
    std::ifstream f(path);
    if (!f) return fail(QBG_E_TABLE, std::string("cannot open ") + path + ": " + std::strerror(errno));
    std::string line;
    if (!std::getline(f, line)) return fail(QBG_E_TABLE, "empty table");
    int version = 0;
    {
        std::istringstream h(line);
        std::string magic, arch;
        if (!(h >> magic >> version >> arch) || magic != "qbg-config-table" ||
            version < 1 || version > 3)
            return fail(QBG_E_TABLE, "bad header (want 'qbg-config-table 1|2|3 <arch>')");
        if (arch != "gfx950") return fail(QBG_E_TABLE, "table is for " + arch + ", not gfx950");
    }
    const int nfields = version + 6;  // v2 adds rotate, v3 the fuse mode
    auto t = std::make_shared<Table>();
    int lineno = 1;
    while (std::getline(f, line)) {
        ++lineno;
        const size_t hash = line.find('#');
        if (hash != std::string::npos) line.resize(hash);
        std::istringstream in(line);
        std::string opname;
        if (!(in >> opname)) continue;  // blank or comment
        int64_t mb, n, k;
        int kid, swap, split, rotate = 0, fuse = 0;
        std::string extra;
        bool okf = static_cast<bool>(in >> mb >> n >> k >> kid >> swap >> split);
        if (okf && version >= 2) okf = static_cast<bool>(in >> rotate);
        if (okf && version >= 3) okf = static_cast<bool>(in >> fuse);
        if (!okf || (in >> extra))
            return fail(QBG_E_TABLE, "line " + std::to_string(lineno) + ": want " +
                                         std::to_string(nfields) + " fields");
        const int op = op_from_name(opname);
        if (op < 0) return fail(QBG_E_TABLE, "line " + std::to_string(lineno) + ": unknown op " + opname);
        if (!is_pow2(mb) || mb > kMaxGroupedRows || n < 16 || n % 16 || k < 16 || k % 16)
            return fail(QBG_E_TABLE, "line " + std::to_string(lineno) + ": bad shape");
        qbg_gemm_config c{};
        c.kernel_id = kid;
        c.swap_ab = swap;
        c.split_k = split;
        c.rotate = rotate;
        c.fuse = fuse;
        if (check_config(op, k, c) != QBG_OK)
            return fail(QBG_E_TABLE, "line " + std::to_string(lineno) + ": " + g_last_error);
        (*t)[Key{op, mb, n, k}] = Entry{kid, swap, split, rotate, fuse};
    }
    std::atomic_store(&g_table, std::shared_ptr<const Table>(t));
    g_table_installed.store(true);
    return ok();
}

}  // namespace

extern "C" {

int qbg_abi_version(void) { return QBG_ABI_VERSION; }

const char* qbg_status_str(qbg_status s_arg) {
    switch (raw_enum(s_arg)) {
        case QBG_OK: return "ok";
        case QBG_E_NULL: return "null pointer";
        case QBG_E_SHAPE: return "bad shape";
        case QBG_E_ALIGN: return "misaligned pointer";
        case QBG_E_QTYPE: return "unknown type, scale format or op";
        case QBG_E_SPLITK: return "infeasible split_k";
        case QBG_E_WORKSPACE: return "workspace missing or too small";
        case QBG_E_TABLE: return "configuration table error";
        case QBG_E_HIP: return "HIP runtime error";
        case QBG_E_CONFIG: return "bad configuration";
    }
    return "unknown status";
}

const char* qbg_last_error(void) { return g_last_error.c_str(); }

qbg_status qbg_quantize_per_token(qbg_qtype qtype_arg, const void* x, int64_t M, int64_t K, void* q,
                                  float* scale, void* stream) {
    const int qtype_v = raw_enum(qtype_arg);
    if (qtype_v != QBG_FP8_E4M3 && qtype_v != QBG_INT8) return fail(QBG_E_QTYPE, "unknown qtype");
    const qbg_qtype qtype = static_cast<qbg_qtype>(qtype_v);
    if (!x || !q || !scale) return fail(QBG_E_NULL, "null pointer");
    if (M < 1 || M > kMaxRows || K < 16 || K % 16 != 0 || K > kMaxDim)
        return fail(QBG_E_SHAPE, "need M in [1, 2^22] and K a positive multiple of 16");
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4))
        return fail(QBG_E_ALIGN, "x and q must be 16-byte aligned, scale 4-byte aligned");
    return hip_status(qbg::launch_quant_per_token((int)qtype, x, M, K, q, scale,
                                                  static_cast<hipStream_t>(stream)),
                      "quantize_per_token launch");
}

qbg_status qbg_quantize_per_token_group(const void* x, int64_t M, int64_t K, int32_t group,
                                        qbg_scale_fmt fmt_arg, void* q, void* scale, void* stream) {
    const int fmt_v = raw_enum(fmt_arg);
    if (fmt_v != QBG_SCALE_F32 && fmt_v != QBG_SCALE_UE8M0) return fail(QBG_E_QTYPE, "unknown scale format");
    const qbg_scale_fmt fmt = static_cast<qbg_scale_fmt>(fmt_v);
    if (!x || !q || !scale) return fail(QBG_E_NULL, "null pointer");
    if (group != 128) return fail(QBG_E_SHAPE, "group must be 128");
    if (M < 1 || M > kMaxDim || K < 128 || K % 128 != 0 || K > kMaxDim || M * (K / 128) > kMaxGroups)
        return fail(QBG_E_SHAPE, "need M >= 1, K a positive multiple of 128 and M*K/128 <= 2^27");
    if (!aligned(x, 16) || !aligned(q, 16) || (fmt == QBG_SCALE_F32 && !aligned(scale, 4)))
        return fail(QBG_E_ALIGN, "x and q must be 16-byte aligned, fp32 scales 4-byte aligned");
    return hip_status(qbg::launch_quant_group(x, M, K, fmt == QBG_SCALE_UE8M0, q, scale,
                                              static_cast<hipStream_t>(stream)),
                      "quantize_per_token_group launch");
}

qbg_status qbg_quantize_weight_block(const void* w, int64_t N, int64_t K, qbg_scale_fmt fmt_arg,
                                     void* q, void* scale, void* stream) {
    const int fmt_v = raw_enum(fmt_arg);
    if (fmt_v != QBG_SCALE_F32 && fmt_v != QBG_SCALE_UE8M0) return fail(QBG_E_QTYPE, "unknown scale format");
    const qbg_scale_fmt fmt = static_cast<qbg_scale_fmt>(fmt_v);
    if (!w || !q || !scale) return fail(QBG_E_NULL, "null pointer");
    if (N < 16 || N % 16 != 0 || N > kMaxDim || K < 128 || K % 128 != 0 || K > kMaxDim)
        return fail(QBG_E_SHAPE, "need N % 16 == 0 and K % 128 == 0");
    if (!aligned(w, 16) || !aligned(q, 16) || (fmt == QBG_SCALE_F32 && !aligned(scale, 4)))
        return fail(QBG_E_ALIGN, "w and q must be 16-byte aligned, fp32 scales 4-byte aligned");
    return hip_status(qbg::launch_quant_weight_block(w, N, K, fmt == QBG_SCALE_UE8M0, q, scale,
                                                     static_cast<hipStream_t>(stream)),
                      "quantize_weight_block launch");
}

qbg_status qbg_rms_norm_quantize_per_token(const void* x, const void* w, float eps, int64_t M,
                                           int64_t H, void* q, float* scale, void* stream) {
    if (!x || !w || !q || !scale) return fail(QBG_E_NULL, "null pointer");
    if (M < 1 || M > kMaxRows || H < 16 || H % 16 != 0 || !qbg::rows_fit_registers(H))
        return fail(QBG_E_SHAPE, "need M >= 1 and H a multiple of 16, at most 65536");
    if (!(eps > 0.0f) || eps == INFINITY) return fail(QBG_E_SHAPE, "eps must be positive and finite");
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) || !aligned(scale, 4))
        return fail(QBG_E_ALIGN, "x, w and q must be 16-byte aligned, scale 4-byte aligned");
    return hip_status(qbg::launch_rms_norm_quant(x, w, eps, M, H, 0, q, scale,
                                                 static_cast<hipStream_t>(stream)),
                      "rms_norm_quantize launch");
}

qbg_status qbg_rms_norm_quantize_per_token_group(const void* x, const void* w, float eps,
                                                 int64_t M, int64_t H, int32_t group,
                                                 qbg_scale_fmt fmt_arg, void* q, void* scale,
                                                 void* stream) {
    const int fmt_v = raw_enum(fmt_arg);
    if (fmt_v != QBG_SCALE_F32 && fmt_v != QBG_SCALE_UE8M0) return fail(QBG_E_QTYPE, "unknown scale format");
    const qbg_scale_fmt fmt = static_cast<qbg_scale_fmt>(fmt_v);
    if (!x || !w || !q || !scale) return fail(QBG_E_NULL, "null pointer");
    if (group != 128) return fail(QBG_E_SHAPE, "group must be 128");
    if (M < 1 || M > kMaxRows || H < 128 || H % 128 != 0 || !qbg::rows_fit_registers(H))
        return fail(QBG_E_SHAPE, "need M >= 1 and H a multiple of 128, at most 65536");
    if (!(eps > 0.0f) || eps == INFINITY) return fail(QBG_E_SHAPE, "eps must be positive and finite");
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) ||
        !aligned(scale, fmt == QBG_SCALE_F32 ? 4 : 1))
        return fail(QBG_E_ALIGN, "x, w and q must be 16-byte aligned, fp32 scales 4-byte aligned");
    return hip_status(qbg::launch_rms_norm_quant(x, w, eps, M, H, fmt == QBG_SCALE_F32 ? 1 : 2, q,
                                                 scale, static_cast<hipStream_t>(stream)),
                      "rms_norm_quantize_per_token_group launch");
}

qbg_status qbg_silu_mul_quantize_per_token(const void* gate_up, int64_t M, int64_t I, void* q,
                                           float* scale, void* stream) {
    if (!gate_up || !q || !scale) return fail(QBG_E_NULL, "null pointer");
    if (M < 1 || M > kMaxRows || I < 16 || I % 16 != 0 || !qbg::rows_fit_registers(I))
        return fail(QBG_E_SHAPE, "need M >= 1 and I a multiple of 16, at most 65536");
    if (!aligned(gate_up, 16) || !aligned(q, 16) || !aligned(scale, 4))
        return fail(QBG_E_ALIGN, "gate_up and q must be 16-byte aligned, scale 4-byte aligned");
    return hip_status(qbg::launch_silu_mul_quant(gate_up, M, I, 0, q, scale,
                                                 static_cast<hipStream_t>(stream)),
                      "silu_mul_quantize launch");
}

qbg_status qbg_silu_mul_quantize_per_token_group(const void* gate_up, int64_t M, int64_t I,
                                                 int32_t group, qbg_scale_fmt fmt_arg, void* q,
                                                 void* scale, void* stream) {
    const int fmt_v = raw_enum(fmt_arg);
    if (fmt_v != QBG_SCALE_F32 && fmt_v != QBG_SCALE_UE8M0) return fail(QBG_E_QTYPE, "unknown scale format");
    const qbg_scale_fmt fmt = static_cast<qbg_scale_fmt>(fmt_v);
    if (!gate_up || !q || !scale) return fail(QBG_E_NULL, "null pointer");
    if (group != 128) return fail(QBG_E_SHAPE, "group must be 128");
    if (M < 1 || M > kMaxRows || I < 128 || I % 128 != 0 || !qbg::rows_fit_registers(I))
        return fail(QBG_E_SHAPE, "need M >= 1 and I a multiple of 128, at most 65536");
    if (!aligned(gate_up, 16) || !aligned(q, 16) || !aligned(scale, fmt == QBG_SCALE_F32 ? 4 : 1))
        return fail(QBG_E_ALIGN, "gate_up and q must be 16-byte aligned, fp32 scales 4-byte aligned");
    return hip_status(qbg::launch_silu_mul_quant(gate_up, M, I, fmt == QBG_SCALE_F32 ? 1 : 2, q,
                                                 scale, static_cast<hipStream_t>(stream)),
                      "silu_mul_quantize_per_token_group launch");
}

qbg_status qbg_convert_f32_to_e4m3(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (n < 0 || n > kMaxDim) return fail(QBG_E_SHAPE, "n out of range");
    if (n > 0 && (!in || !out)) return fail(QBG_E_NULL, "null pointer");
    if (!aligned(in, 4)) return fail(QBG_E_ALIGN, "in must be 4-byte aligned");
    return hip_status(qbg::launch_convert_e4m3(in, out, n, static_cast<hipStream_t>(stream)),
                      "convert launch");
}

qbg_status qbg_scaled_mm(qbg_qtype qtype_arg, const void* a_q, const float* a_scale, const void* w_q,
                         const float* w_scale, int64_t M, int64_t N, int64_t K, void* out,
                         const qbg_gemm_config* cfg, void* workspace, size_t workspace_bytes,
                         void* stream) {
    const int qtype_v = raw_enum(qtype_arg);
    if (qtype_v != QBG_FP8_E4M3 && qtype_v != QBG_INT8) return fail(QBG_E_QTYPE, "unknown qtype");
    const qbg_qtype qtype = static_cast<qbg_qtype>(qtype_v);
    const int op = qtype == QBG_FP8_E4M3 ? QBG_OP_FP8 : QBG_OP_INT8;
    return run_gemm(op, a_q, a_scale, w_q, w_scale, M, N, K, out, 0, cfg, workspace,
                    workspace_bytes, stream);
}

qbg_status qbg_scaled_mm_noalloc(qbg_qtype qtype_arg, const void* a_q, const float* a_scale,
                                 const void* w_q, const float* w_scale, int64_t M, int64_t N,
                                 int64_t K, void* out, const qbg_gemm_config* cfg, void* stream) {
    const int qtype_v = raw_enum(qtype_arg);
    if (qtype_v != QBG_FP8_E4M3 && qtype_v != QBG_INT8) return fail(QBG_E_QTYPE, "unknown qtype");
    const qbg_qtype qtype = static_cast<qbg_qtype>(qtype_v);
    const int op = qtype == QBG_FP8_E4M3 ? QBG_OP_FP8 : QBG_OP_INT8;
    return run_gemm(op, a_q, a_scale, w_q, w_scale, M, N, K, out, 0, cfg, nullptr, 0, stream,
                    nullptr, true);
}

qbg_status qbg_block_scaled_mm(qbg_scale_fmt fmt_arg, const void* a_q, const void* a_scale,
                               const void* w_q, const void* w_scale, int64_t M, int64_t N,
                               int64_t K, void* out, const qbg_gemm_config* cfg, void* workspace,
                               size_t workspace_bytes, void* stream) {
    const int fmt_v = raw_enum(fmt_arg);
    if (fmt_v != QBG_SCALE_F32 && fmt_v != QBG_SCALE_UE8M0) return fail(QBG_E_QTYPE, "unknown scale format");
    const qbg_scale_fmt fmt = static_cast<qbg_scale_fmt>(fmt_v);
    const int op = fmt == QBG_SCALE_F32 ? QBG_OP_BLOCK_FP8 : QBG_OP_BLOCK_UE8M0;
    return run_gemm(op, a_q, a_scale, w_q, w_scale, M, N, K, out, 0, cfg, workspace,
                    workspace_bytes, stream);
}

qbg_status qbg_quantize_scaled_mm(qbg_qtype qtype_arg, const void* x, const void* w_q,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* a_q,
                                  float* a_scale, void* out, const qbg_gemm_config* cfg,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    const int qtype_v = raw_enum(qtype_arg);
    if (qtype_v != QBG_FP8_E4M3 && qtype_v != QBG_INT8) return fail(QBG_E_QTYPE, "unknown qtype");
    const qbg_qtype qtype = static_cast<qbg_qtype>(qtype_v);
    const int op = qtype == QBG_FP8_E4M3 ? QBG_OP_FP8_FUSED : QBG_OP_INT8_FUSED;
    return run_gemm(op, a_q, a_scale, w_q, w_scale, M, N, K, out, 0, cfg, workspace,
                    workspace_bytes, stream, x);
}

int32_t qbg_set_fused_wait_limit(int32_t iterations) {
    return g_wait_limit.exchange(iterations < 0 ? qbg::kDefaultWaitLimit : iterations);
}

qbg_status qbg_grouped_scaled_mm(qbg_qtype qtype_arg, const void* a_q, const float* a_scale,
                                 const void* w_q, const float* w_scale, const int32_t* offsets,
                                 int64_t T, int64_t E, int64_t N, int64_t K, void* out,
                                 const qbg_gemm_config* cfg, void* stream) {
    const int qtype_v = raw_enum(qtype_arg);
    if (qtype_v != QBG_FP8_E4M3 && qtype_v != QBG_INT8) return fail(QBG_E_QTYPE, "unknown qtype");
    const qbg_qtype qtype = static_cast<qbg_qtype>(qtype_v);
    const int op = qtype == QBG_FP8_E4M3 ? QBG_OP_FP8_GROUPED : QBG_OP_INT8_GROUPED;
    if (T < 0 || T > kMaxGroupedRows) return fail(QBG_E_SHAPE, "T must be in [0, 65536]");
    if (E < 1 || E > kMaxExperts) return fail(QBG_E_SHAPE, "E must be in [1, 65535]");
    qbg_status st = check_gemm_shape(1, N, K);
    if (st != QBG_OK) return st;
    if (!a_q || !a_scale || !w_q || !w_scale || !offsets || !out)
        return fail(QBG_E_NULL, "null tensor pointer");
    if (!aligned(a_q, 16) || !aligned(w_q, 16)) return fail(QBG_E_ALIGN, "operands must be 16-byte aligned");
    if (!aligned(a_scale, 4) || !aligned(w_scale, 4) || !aligned(offsets, 4) || !aligned(out, 4))
        return fail(QBG_E_ALIGN, "scales, offsets and out must be 4-byte aligned");
    int from_table = 0;
    qbg_gemm_config c = resolve(op, T > 0 ? T : 1, N, K, cfg, &from_table);
    // No table entry and at least 32 routed rows per expert on average: the
    // 64-token prefill tile (its token tiles are then mostly full)
    if (!cfg && !from_table && T >= 32 * E && K % 128 == 0 && E <= kMaxPrefillExperts) {
        for (int k = 0; k < qbg::gemm_kernel_count(); ++k) {
            const qbg::TileShape t = qbg::gemm_tile(k);
            if (t.big > 0 && t.tm == 64 && qbg::tile_n(t) == 128) {
                c = qbg_gemm_config{};
                c.kernel_id = k;
                c.split_k = 1;
                fill_tile(&c);
                break;
            }
        }
    }
    // A looked-up prefill tile with more experts than its offset scan takes: the
    // decode tiles' default instead (a forced configuration is rejected below).
    if (!cfg && qbg::gemm_tile(c.kernel_id).big > 0 && E > kMaxPrefillExperts) {
        const Entry e = default_config(op, T > 0 ? T : 1, N, K);
        c = qbg_gemm_config{};
        c.kernel_id = e.kernel_id;
        c.swap_ab = e.swap_ab;
        c.split_k = e.split_k;
        c.rotate = e.rotate;
        fill_tile(&c);
    }
    st = check_config(op, K, c);
    if (st != QBG_OK) return st;
    if (qbg::gemm_tile(c.kernel_id).big > 0 && E > kMaxPrefillExperts)
        return fail(QBG_E_CONFIG, "grouped GEMMs on the prefill tiles take at most " +
                                      std::to_string(kMaxPrefillExperts) + " experts");
    st = check_lds(op, std::min<int64_t>(T > 0 ? T : 1, qbg::kMaxTokensPerLaunch), K, c);
    if (st != QBG_OK) return st;
    if (T == 0) return ok();  // no routed rows: nothing to compute
    if (log_enabled())
        std::fprintf(stderr, "[qbg] grouped op=%d T=%lld E=%lld N=%lld K=%lld kernel=%d swap_ab=%d\n",
                     op, (long long)T, (long long)E, (long long)N, (long long)K, c.kernel_id,
                     c.swap_ab);
    qbg::GemmArgs p{};
    p.a = static_cast<const uint8_t*>(a_q);
    p.a_scale = a_scale;
    p.w = static_cast<const uint8_t*>(w_q);
    p.w_scale = w_scale;
    p.out = out;
    p.M = (int)std::min<int64_t>(T, qbg::kMaxTokensPerLaunch);
    p.N = (int)N;
    p.K = (int)K;
    p.k_chunk = (int)K;
    p.split_k = 1;
    p.kgroups = (int)(K / 128);
    p.rotate = c.rotate;
    p.offsets = offsets;
    p.experts = (int)E;
    p.rows = (int)T;
    return hip_status(qbg::launch_gemm(op, p, c.kernel_id, c.swap_ab, static_cast<hipStream_t>(stream)),
                      "grouped GEMM launch");
}

qbg_status qbg_scaled_mm_i32(const void* a_q, const void* w_q, int64_t M, int64_t N, int64_t K,
                             int32_t* acc, const qbg_gemm_config* cfg, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return run_gemm(QBG_OP_INT8, a_q, nullptr, w_q, nullptr, M, N, K, acc, 1, cfg, workspace,
                    workspace_bytes, stream);
}

qbg_status qbg_config_table_load(const char* path) {
    const qbg_status st = load_table_file(path);
    if (st == QBG_OK) g_table_installed.store(true);
    return st;
}


int64_t qbg_config_table_size(void) {
    autoload_table();
    std::shared_ptr<const Table> t = std::atomic_load(&g_table);
    return t ? (int64_t)t->size() : 0;
}

qbg_status qbg_config_lookup(qbg_op op_arg, int64_t M, int64_t N, int64_t K, qbg_gemm_config* out,
                             int32_t* from_table) {
    const int op = raw_enum(op_arg);
    if (!op_valid(op)) return fail(QBG_E_QTYPE, "unknown op");
    if (!out) return fail(QBG_E_NULL, "null output");
    qbg_status st = is_grouped(op) ? check_gemm_shape(1, N, K) : check_gemm_shape(M, N, K);
    if (st == QBG_OK && is_grouped(op) && (M < 1 || M > kMaxGroupedRows))
        st = fail(QBG_E_SHAPE, "grouped rows must be in [1, 65536]");
    if (st != QBG_OK) return st;
    int hit = 0;
    *out = resolve(op, M, N, K, nullptr, &hit);
    if (from_table) *from_table = hit;
    return ok();
}

qbg_status qbg_workspace_size(qbg_op op_arg, int64_t M, int64_t N, int64_t K,
                              const qbg_gemm_config* cfg, size_t* bytes) {
    const int op = raw_enum(op_arg);
    if (!op_valid(op)) return fail(QBG_E_QTYPE, "unknown op");
    if (!bytes) return fail(QBG_E_NULL, "null output");
    qbg_status st = is_grouped(op) ? check_gemm_shape(1, N, K) : check_gemm_shape(M, N, K);
    if (st == QBG_OK && is_grouped(op) && (M < 1 || M > kMaxGroupedRows))
        st = fail(QBG_E_SHAPE, "grouped rows must be in [1, 65536]");
    if (st != QBG_OK) return st;
    const qbg_gemm_config c = resolve(op, M, N, K, cfg, nullptr);
    st = check_config(op, K, c);
    if (st != QBG_OK) return st;
    st = check_lds(op, is_grouped(op) ? std::min<int64_t>(M, qbg::kMaxTokensPerLaunch) : M, K, c);
    if (st != QBG_OK) return st;
    *bytes = workspace_bytes(op, M, N, c);
    return ok();
}

qbg_status qbg_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (workspace_bytes == 0) return ok();
    if (!workspace) return fail(QBG_E_NULL, "null workspace");
    if (!aligned(workspace, 4)) return fail(QBG_E_ALIGN, "workspace must be 4-byte aligned");
    return hip_status(qbg::launch_fill_zero(workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
                      "workspace fill");
}

int32_t qbg_kernel_count(void) { return qbg::gemm_kernel_count(); }

qbg_status qbg_kernel_info(int32_t kernel_id, qbg_gemm_config* inout) {
    if (!inout) return fail(QBG_E_NULL, "null output");
    if (kernel_id < 0 || kernel_id >= qbg::gemm_kernel_count())
        return fail(QBG_E_CONFIG, "kernel_id out of range");
    inout->kernel_id = kernel_id;
    fill_tile(inout);
    return ok();
}

}  // extern "C"
