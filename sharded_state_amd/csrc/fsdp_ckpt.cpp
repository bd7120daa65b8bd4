// fsdp_ckpt.cpp -- sharded-state checkpoint files of libfsdp_shard.so.
//
// "fairseq 中的 Fully Sharded Data Parallel (FSDP) 实战指南" (zskr.cn), section
// "工作原理", checkpoint paragraph: with --use-sharded-state every rank saves
// its own local state to a file whose name carries the suffix -shard{rank}, and
// loads it back the same way; the default mode instead consolidates the full
// state on one rank.  "FSDP (Fully Sharded Data Parallel)" (vanos001 notes),
// section "FSDP Checkpointing": sharded state dicts saved and loaded per rank.
//
// File layout (little-endian):
//   [0, 256)            header (FileHeader below)
//   [256, 256 + 8*T)    the unit's tensor sizes (int64 numels, flat order)
//   [payload_offset..)  master, exp_avg, exp_avg_sq shards, S elements each of the
//                       state dtype, back to back; payload_offset is 4096-aligned
//                       and the file ends with the payload
// The header carries CRC32C (Castagnoli) checksums of itself (with its own
// checksum field zero), of the size table and of the payload; a reader checks
// every size and offset against the file's length before it allocates or seeks.  A file is written to "<path>.tmp", flushed, synced and renamed, so a
// reader never sees a partial file under the final name.  Device buffers move
// through two pinned host staging buffers: the copy of chunk k+1 overlaps the
// file write of chunk k (save) or the file read of chunk k+1 overlaps the copy
// of chunk k (load).  A save checksums each chunk on a helper thread beside its
// write; a load reads and checksums each chunk in parts on the worker pool.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <future>
#include <thread>
#include <cerrno>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include "fsdp_internal.h"
#include "fsdp_pool.h"
#include "fsdp_shard.h"

namespace {

using fsdp::Pool;

constexpr char kMagic[8] = {'F', 'S', 'D', 'P', 'S', 'H', 'R', 'D'};
constexpr uint32_t kVersion = 2;   // 2: the header checksums itself
constexpr uint64_t kAlign = 4096;
constexpr size_t kChunk = 32u << 20;   // staging chunk

struct FileHeader {
    char magic[8];
    uint32_t version;
    uint32_t header_bytes;
    int32_t world;
    int32_t rank;
    int64_t numel;
    int64_t padded_numel;
    int64_t shard_numel;
    int32_t state_dt;
    int32_t compute_dt;
    int64_t step;
    float lr, beta1, beta2, eps, weight_decay;
    int32_t n_tensors;
    uint64_t payload_offset;
    uint64_t payload_bytes;
    uint32_t crc_table;
    uint32_t crc_payload;
    uint32_t crc_header;   // CRC32C of the 256 header bytes with this field zero
    uint8_t reserved[256 - 116];
};
static_assert(sizeof(FileHeader) == 256, "header is 256 bytes");

// ------------------------------------------------------------------ CRC32C
// Castagnoli polynomial 0x1EDC6F41 (reflected 0x82F63B78), initial value and
// final xor 0xFFFFFFFF.  SSE4.2 has the instruction; a table covers other hosts.
uint32_t g_crc_table[8][256];

void crc_init_table() {
    for (uint32_t i = 0; i < 256; ++i) {
        uint32_t c = i;
        for (int k = 0; k < 8; ++k) c = (c & 1) ? (c >> 1) ^ 0x82F63B78u : (c >> 1);
        g_crc_table[0][i] = c;
    }
    for (int t = 1; t < 8; ++t)
        for (uint32_t i = 0; i < 256; ++i)
            g_crc_table[t][i] = (g_crc_table[t - 1][i] >> 8) ^ g_crc_table[0][g_crc_table[t - 1][i] & 0xff];
}

uint32_t crc_soft(uint32_t crc, const unsigned char* p, size_t n) {
    // thread-safe one-time set-up: a save's helper thread and its caller may both get here first
    static const bool ready = (crc_init_table(), true);
    (void)ready;
    while (n >= 8) {
        uint64_t w;
        memcpy(&w, p, 8);
        w ^= crc;
        crc = g_crc_table[7][w & 0xff] ^ g_crc_table[6][(w >> 8) & 0xff] ^ g_crc_table[5][(w >> 16) & 0xff] ^
              g_crc_table[4][(w >> 24) & 0xff] ^ g_crc_table[3][(w >> 32) & 0xff] ^
              g_crc_table[2][(w >> 40) & 0xff] ^ g_crc_table[1][(w >> 48) & 0xff] ^ g_crc_table[0][w >> 56];
        p += 8;
        n -= 8;
    }
    while (n--) crc = (crc >> 8) ^ g_crc_table[0][(crc ^ *p++) & 0xff];
    return crc;
}

__attribute__((target("sse4.2"))) uint32_t crc_hw(uint32_t crc, const unsigned char* p, size_t n) {
    uint64_t c = crc;
    while (n >= 8) {
        uint64_t w;
        memcpy(&w, p, 8);
        c = __builtin_ia32_crc32di(c, w);
        p += 8;
        n -= 8;
    }
    uint32_t c32 = (uint32_t)c;
    while (n--) c32 = __builtin_ia32_crc32qi(c32, *p++);
    return c32;
}

// The CRC register update is linear over GF(2): running it over `n` zero bytes
// maps a register value x to Z_n(x) for a fixed 32x32 bit matrix Z_n.  So for
// two consecutive blocks A, B:  reg(s, A || B) = Z_|B|(reg(s, A)) ^ reg(0, B),
// which lets independent chains over parts of a buffer be combined.
struct Gf2Matrix {
    uint32_t col[32];   // col[i] = image of the register value with only bit i set
};

uint32_t gf2_apply(const Gf2Matrix& m, uint32_t v) {
    uint32_t r = 0;
    for (int i = 0; v; ++i, v >>= 1)
        if (v & 1) r ^= m.col[i];
    return r;
}

Gf2Matrix gf2_mul(const Gf2Matrix& a, const Gf2Matrix& b) {   // a after b
    Gf2Matrix r;
    for (int i = 0; i < 32; ++i) r.col[i] = gf2_apply(a, b.col[i]);
    return r;
}

// Z_n: the register map of n zero bytes (reflected polynomial 0x82F63B78).
Gf2Matrix zero_bytes_map(uint64_t n) {
    Gf2Matrix bit;   // one zero bit: x -> (x >> 1) ^ (x & 1 ? poly : 0)
    bit.col[0] = 0x82F63B78u;
    for (int i = 1; i < 32; ++i) bit.col[i] = 1u << (i - 1);
    Gf2Matrix byte = bit;
    for (int k = 0; k < 3; ++k) byte = gf2_mul(byte, byte);   // 8 zero bits
    Gf2Matrix r;
    for (int i = 0; i < 32; ++i) r.col[i] = 1u << i;          // identity
    while (n) {
        if (n & 1) r = gf2_mul(byte, r);
        byte = gf2_mul(byte, byte);
        n >>= 1;
    }
    return r;
}

// Three independent hardware chains over thirds of the buffer (the crc32
// instruction's latency is three times its issue interval), combined with Z.
__attribute__((target("sse4.2"))) uint32_t crc_hw3(uint32_t crc, const unsigned char* p, size_t n) {
    const size_t lane = (n / 3) & ~(size_t)7;
    const unsigned char* pb = p + lane;
    const unsigned char* pc = p + 2 * lane;
    uint64_t a = crc, b = 0, c = 0;
    for (size_t off = 0; off < lane; off += 8) {
        uint64_t wa, wb, wc;
        memcpy(&wa, p + off, 8);
        memcpy(&wb, pb + off, 8);
        memcpy(&wc, pc + off, 8);
        a = __builtin_ia32_crc32di(a, wa);
        b = __builtin_ia32_crc32di(b, wb);
        c = __builtin_ia32_crc32di(c, wc);
    }
    const uint32_t c_rest = crc_hw((uint32_t)c, pc + lane, n - 3 * lane);   // lane C's tail
    const size_t len_c = n - 2 * lane;
    thread_local uint64_t z_len[2] = {~0ull, ~0ull};
    thread_local Gf2Matrix z[2];
    const uint64_t want[2] = {lane, len_c};
    for (int k = 0; k < 2; ++k)
        if (z_len[k] != want[k]) {
            z[k] = zero_bytes_map(want[k]);
            z_len[k] = want[k];
        }
    const uint32_t ab = gf2_apply(z[0], (uint32_t)a) ^ (uint32_t)b;
    return gf2_apply(z[1], ab) ^ c_rest;
}

// Continue a CRC32C over n more bytes (state: the running value before the final xor).
uint32_t crc_update(uint32_t state, const void* data, size_t n) {
    static const bool hw = __builtin_cpu_supports("sse4.2");
    const unsigned char* p = (const unsigned char*)data;
    if (!hw) return crc_soft(state, p, n);
    return n >= (64u << 10) ? crc_hw3(state, p, n) : crc_hw(state, p, n);
}

// ------------------------------------------------------------------ parallel reads
// A buffered read of one file scales with threads (a write does not: the
// kernel serialises writes to one file), so the reader splits the payload into
// parts of at least kPartMin bytes, each read with pread and checksummed from
// a zero register by one worker of the pool; the parts' registers are then
// folded in file order with the zero-bytes map: reg(s, A || B) = Z_|B|(reg(s,
// A)) ^ reg(0, B).
constexpr size_t kPartMin = 4u << 20;

int read_threads() {
    static const int n = [] {
        const unsigned hc = std::thread::hardware_concurrency();
        return (int)std::max(1u, std::min(hc ? hc : 1u, 8u));
    }();
    return n;
}

bool pread_all(int fd, char* dst, size_t n, uint64_t off) {
    while (n) {
        const ssize_t r = pread(fd, dst, n, (off_t)off);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        dst += r;
        n -= (size_t)r;
        off += (uint64_t)r;
    }
    return true;
}

// Z_n for the part lengths of the last calls (at most two distinct lengths per call).
const Gf2Matrix& zero_map_cached(uint64_t n) {
    thread_local uint64_t len[2] = {~0ull, ~0ull};
    thread_local Gf2Matrix z[2];
    thread_local int next = 0;
    for (int k = 0; k < 2; ++k)
        if (len[k] == n) return z[k];
    const int k = next;
    next ^= 1;
    z[k] = zero_bytes_map(n);
    len[k] = n;
    return z[k];
}

// Read n bytes at file offset `off` into dst and advance the running CRC32C
// register `state` over them.  false on a short read or a read error.
bool read_sum(int fd, uint64_t off, char* dst, size_t n, uint32_t& state) {
    if (n == 0) return true;
    const int parts = (int)std::max<size_t>(1, std::min<size_t>((size_t)read_threads(), n / kPartMin));
    const size_t per = (n + parts - 1) / parts;
    std::vector<uint32_t> reg(parts, 0u);
    std::atomic<bool> ok{true};
    Pool::get().run_workers(parts, [&](int w) {
        const size_t lo = (size_t)w * per, hi = std::min(n, lo + per);
        if (lo >= hi) return;
        if (!pread_all(fd, dst + lo, hi - lo, off + lo)) {
            ok.store(false);
            return;
        }
        reg[w] = crc_update(0u, dst + lo, hi - lo);
    });
    if (!ok.load()) return false;
    for (int w = 0; w < parts; ++w) {
        const size_t lo = (size_t)w * per, hi = std::min(n, lo + per);
        if (lo >= hi) break;
        state = gf2_apply(zero_map_cached(hi - lo), state) ^ reg[w];
    }
    return true;
}

// ------------------------------------------------------------------ staging
// Two pinned host buffers, allocated per call and freed on every exit path.
struct Staging {
    void* buf[2] = {nullptr, nullptr};
    hipEvent_t ev[2] = {nullptr, nullptr};
    ~Staging() {
        // copies may still be in flight on an error path: wait before freeing
        for (int i = 0; i < 2; ++i)
            if (ev[i]) (void)hipEventSynchronize(ev[i]);
        for (int i = 0; i < 2; ++i) {
            if (ev[i]) (void)hipEventDestroy(ev[i]);
            if (buf[i]) (void)hipHostFree(buf[i]);
        }
    }
    hipError_t init() {
        for (int i = 0; i < 2; ++i) {
            hipError_t e = hipHostMalloc(&buf[i], kChunk, hipHostMallocDefault);
            if (e != hipSuccess) return e;
            e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
};

struct File {
    FILE* f = nullptr;
    ~File() {
        if (f) fclose(f);
    }
};

bool write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n; }
bool read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

// One contiguous piece of the payload: the bytes of one state buffer.
struct Piece {
    const char* src;   // save: source; load: unused
    char* dst;         // load: destination
    uint64_t bytes;
};

// Largest shard a file may describe: three shards of 4-byte elements stay far
// inside 64-bit byte counts.
constexpr int64_t kMaxShard = INT64_MAX / 64;

int check_info(const fsdp_ckpt_info* in) {
    if (!in) return fsdp::fail(FSDP_E_INVAL, "info is NULL");
    if (in->world < 1 || in->rank < 0 || in->rank >= in->world)
        return fsdp::fail(FSDP_E_INVAL, "world %d / rank %d out of range", in->world, in->rank);
    if (in->numel < 0 || in->padded_numel < in->numel || in->shard_numel < 0 || in->shard_numel > kMaxShard ||
        in->padded_numel % in->world || in->padded_numel / in->world != in->shard_numel)
        return fsdp::fail(FSDP_E_SIZE, "inconsistent sizes: numel %lld, padded %lld, shard %lld, world %d",
                          (long long)in->numel, (long long)in->padded_numel, (long long)in->shard_numel, in->world);
    if (!fsdp::valid_dtype(in->state_dt) || !fsdp::valid_dtype(in->compute_dt))
        return fsdp::fail(FSDP_E_DTYPE, "state dtype %d / compute dtype %d unsupported", in->state_dt, in->compute_dt);
    if (in->n_tensors < 0) return fsdp::fail(FSDP_E_INVAL, "n_tensors < 0");
    return FSDP_OK;
}

uint32_t crc32c(const void* data, uint64_t n) {
    return n ? crc_update(0xFFFFFFFFu, data, (size_t)n) ^ 0xFFFFFFFFu : 0u;
}

// Open a shard file and check its header and size table: magic, version, the
// header's own checksum, consistent sizes, a payload that ends the file
// exactly, the size table's checksum and sum.  Every count read from the file
// is bounded by the file's length before anything is allocated from it.  On
// success the file is open in `in`, positioned after the size table.
int read_header(const char* path, File& in, FileHeader& h, fsdp_ckpt_info& info, std::vector<int64_t>* numels_out) {
    in.f = fopen(path, "rb");
    if (!in.f) return fsdp::fail(FSDP_E_IO, "cannot open %s: %s", path, strerror(errno));
    struct stat sb;
    if (fstat(fileno(in.f), &sb) != 0) return fsdp::fail(FSDP_E_IO, "cannot stat %s: %s", path, strerror(errno));
    const uint64_t file_bytes = (uint64_t)sb.st_size;
    if (!read_all(in.f, &h, sizeof h)) return fsdp::fail(FSDP_E_FORMAT, "%s: truncated header", path);
    if (memcmp(h.magic, kMagic, 8) != 0) return fsdp::fail(FSDP_E_FORMAT, "%s: not a shard file", path);
    if (h.version != kVersion || h.header_bytes != sizeof(FileHeader))
        return fsdp::fail(FSDP_E_FORMAT, "%s: unsupported version %u", path, h.version);
    FileHeader z = h;
    z.crc_header = 0;
    if (crc32c(&z, sizeof z) != h.crc_header) return fsdp::fail(FSDP_E_FORMAT, "%s: header checksum mismatch", path);
    memset(&info, 0, sizeof info);
    info.world = h.world;
    info.rank = h.rank;
    info.numel = h.numel;
    info.padded_numel = h.padded_numel;
    info.shard_numel = h.shard_numel;
    info.state_dt = (fsdp_dtype)h.state_dt;
    info.compute_dt = (fsdp_dtype)h.compute_dt;
    info.step = h.step;
    info.hp.lr = h.lr;
    info.hp.beta1 = h.beta1;
    info.hp.beta2 = h.beta2;
    info.hp.eps = h.eps;
    info.hp.weight_decay = h.weight_decay;
    info.hp.step = h.step;
    info.n_tensors = h.n_tensors;
    if (check_info(&info) != FSDP_OK) return fsdp::fail(FSDP_E_FORMAT, "%s: inconsistent header", path);
    const uint64_t sbytes = (uint64_t)h.shard_numel * (uint64_t)fsdp::dt_size(h.state_dt);   // < 2^58
    const uint64_t table_bytes = 8ull * (uint64_t)h.n_tensors;                                  // < 2^34
    if (h.payload_bytes != 3 * sbytes || h.payload_offset % kAlign != 0 ||
        h.payload_offset < sizeof(FileHeader) + table_bytes || h.payload_offset > file_bytes ||
        file_bytes - h.payload_offset != h.payload_bytes)
        return fsdp::fail(FSDP_E_FORMAT, "%s: payload layout does not match the file's %llu bytes", path,
                          (unsigned long long)file_bytes);
    std::vector<int64_t> numels(h.n_tensors);   // the table lies inside the file: bounded by its length
    if (h.n_tensors && !read_all(in.f, numels.data(), table_bytes))
        return fsdp::fail(FSDP_E_FORMAT, "%s: truncated size table", path);
    if (crc32c(numels.data(), table_bytes) != h.crc_table)
        return fsdp::fail(FSDP_E_FORMAT, "%s: size table checksum mismatch", path);
    int64_t total = 0;
    for (int64_t n : numels)
        if (n < 0 || __builtin_add_overflow(total, n, &total))
            return fsdp::fail(FSDP_E_FORMAT, "%s: invalid size table", path);
    if (total != h.numel) return fsdp::fail(FSDP_E_FORMAT, "%s: size table does not sum to numel", path);
    if (numels_out) numels_out->swap(numels);
    return FSDP_OK;
}

}  // namespace

extern "C" {

uint32_t fsdp_crc32c(const void* data, int64_t n) {
    if (!data || n <= 0) return 0;
    return crc_update(0xFFFFFFFFu, data, (size_t)n) ^ 0xFFFFFFFFu;
}

int fsdp_save_shard(const char* path, const fsdp_ckpt_info* info, const int64_t* numels, const void* master,
                    const void* exp_avg, const void* exp_avg_sq, int32_t on_device, void* stream) {
    int rc = check_info(info);
    if (rc) return rc;
    if (!path || !*path) return fsdp::fail(FSDP_E_INVAL, "path is empty");
    if (info->n_tensors > 0 && !numels) return fsdp::fail(FSDP_E_INVAL, "numels is NULL");
    int64_t total = 0;
    for (int32_t k = 0; k < info->n_tensors; ++k) {
        if (numels[k] < 0) return fsdp::fail(FSDP_E_INVAL, "numels[%d] < 0", k);
        if (__builtin_add_overflow(total, numels[k], &total)) return fsdp::fail(FSDP_E_SIZE, "tensor sizes overflow");
    }
    if (total != info->numel)
        return fsdp::fail(FSDP_E_SIZE, "tensor sizes sum to %lld, info->numel is %lld", (long long)total,
                          (long long)info->numel);
    const uint64_t sbytes = (uint64_t)info->shard_numel * (uint64_t)fsdp::dt_size(info->state_dt);
    if (sbytes > 0 && (!master || !exp_avg || !exp_avg_sq))
        return fsdp::fail(FSDP_E_INVAL, "master, exp_avg and exp_avg_sq must be non-NULL");

    FileHeader h;
    memset(&h, 0, sizeof h);
    memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.header_bytes = sizeof(FileHeader);
    h.world = info->world;
    h.rank = info->rank;
    h.numel = info->numel;
    h.padded_numel = info->padded_numel;
    h.shard_numel = info->shard_numel;
    h.state_dt = info->state_dt;
    h.compute_dt = info->compute_dt;
    h.step = info->step;
    h.lr = info->hp.lr;
    h.beta1 = info->hp.beta1;
    h.beta2 = info->hp.beta2;
    h.eps = info->hp.eps;
    h.weight_decay = info->hp.weight_decay;
    h.n_tensors = info->n_tensors;
    const uint64_t table_bytes = 8ull * (uint64_t)info->n_tensors;
    h.payload_offset = (sizeof(FileHeader) + table_bytes + kAlign - 1) / kAlign * kAlign;
    h.payload_bytes = 3 * sbytes;
    h.crc_table = fsdp_crc32c(numels, (int64_t)table_bytes);

    std::string tmp = std::string(path) + ".tmp";
    File out;
    out.f = fopen(tmp.c_str(), "wb");
    if (!out.f) return fsdp::fail(FSDP_E_IO, "cannot open %s for writing: %s", tmp.c_str(), strerror(errno));
    std::vector<char> pad(h.payload_offset - sizeof(FileHeader) - table_bytes, 0);
    if (!write_all(out.f, &h, sizeof h) || (table_bytes && !write_all(out.f, numels, table_bytes)) ||
        (!pad.empty() && !write_all(out.f, pad.data(), pad.size())))
        return fsdp::fail(FSDP_E_IO, "write to %s failed: %s", tmp.c_str(), strerror(errno));

    const Piece pieces[3] = {{(const char*)master, nullptr, sbytes},
                             {(const char*)exp_avg, nullptr, sbytes},
                             {(const char*)exp_avg_sq, nullptr, sbytes}};
    uint32_t crc = 0xFFFFFFFFu;
    if (on_device) {
        Staging st;
        hipError_t e = st.init();
        if (e != hipSuccess) return fsdp::hip_fail(e, "pinned staging allocation");
        // chunk list over the three pieces; chunk k copies into staging k % 2
        struct Chunk { const char* src; size_t n; };
        std::vector<Chunk> chunks;
        for (const Piece& p : pieces)
            for (uint64_t off = 0; off < p.bytes; off += kChunk)
                chunks.push_back({p.src + off, (size_t)std::min<uint64_t>(kChunk, p.bytes - off)});
        hipStream_t s = (hipStream_t)stream;
        auto issue = [&](size_t k) -> hipError_t {
            hipError_t r = hipMemcpyAsync(st.buf[k % 2], chunks[k].src, chunks[k].n, hipMemcpyDeviceToHost, s);
            if (r == hipSuccess) r = hipEventRecord(st.ev[k % 2], s);
            return r;
        };
        if (!chunks.empty() && (e = issue(0)) != hipSuccess) return fsdp::hip_fail(e, "device-to-host copy");
        for (size_t k = 0; k < chunks.size(); ++k) {
            if ((e = hipEventSynchronize(st.ev[k % 2])) != hipSuccess) return fsdp::hip_fail(e, "device-to-host copy");
            if (k + 1 < chunks.size() && (e = issue(k + 1)) != hipSuccess)
                return fsdp::hip_fail(e, "device-to-host copy");
            // checksum on a helper thread while this thread writes the same bytes
            const void* b = st.buf[k % 2];
            const size_t n = chunks[k].n;
            std::future<uint32_t> sum = std::async(std::launch::async, [crc, b, n] { return crc_update(crc, b, n); });
            const bool wrote = write_all(out.f, b, n);
            crc = sum.get();
            if (!wrote) return fsdp::fail(FSDP_E_IO, "write to %s failed: %s", tmp.c_str(), strerror(errno));
        }
    } else {
        for (const Piece& p : pieces) {
            if (!p.bytes) continue;
            crc = crc_update(crc, p.src, p.bytes);
            if (!write_all(out.f, p.src, p.bytes))
                return fsdp::fail(FSDP_E_IO, "write to %s failed: %s", tmp.c_str(), strerror(errno));
        }
    }
    h.crc_payload = crc ^ 0xFFFFFFFFu;
    h.crc_header = 0;
    h.crc_header = fsdp_crc32c(&h, sizeof h);
    if (fseek(out.f, 0, SEEK_SET) != 0 || !write_all(out.f, &h, sizeof h) || fflush(out.f) != 0 ||
        fsync(fileno(out.f)) != 0)
        return fsdp::fail(FSDP_E_IO, "finishing %s failed: %s", tmp.c_str(), strerror(errno));
    fclose(out.f);
    out.f = nullptr;
    if (rename(tmp.c_str(), path) != 0)
        return fsdp::fail(FSDP_E_IO, "rename %s -> %s failed: %s", tmp.c_str(), path, strerror(errno));
    return fsdp::ok();
}

int fsdp_shard_info(const char* path, fsdp_ckpt_info* info_out, int64_t* numels_out, int32_t numels_capacity) {
    if (!path || !info_out) return fsdp::fail(FSDP_E_INVAL, "path and info_out must be non-NULL");
    File in;
    FileHeader h;
    fsdp_ckpt_info info;
    std::vector<int64_t> numels;
    int rc = read_header(path, in, h, info, &numels);
    if (rc) return rc;
    if (numels_out) {
        if (numels_capacity < h.n_tensors)
            return fsdp::fail(FSDP_E_SIZE, "%s: %d tensors, numels_capacity %d", path, h.n_tensors, numels_capacity);
        if (h.n_tensors) memcpy(numels_out, numels.data(), 8ull * h.n_tensors);
    }
    *info_out = info;
    return fsdp::ok();
}

int fsdp_load_shard(const char* path, fsdp_ckpt_info* info_out, void* master, void* exp_avg, void* exp_avg_sq,
                    int64_t shard_capacity, int32_t on_device, void* stream) {
    if (!path) return fsdp::fail(FSDP_E_INVAL, "path is NULL");
    File in;
    FileHeader h;
    fsdp_ckpt_info info;
    int rc = read_header(path, in, h, info, nullptr);
    if (rc) return rc;
    if (info.shard_numel > shard_capacity)
        return fsdp::fail(FSDP_E_SIZE, "%s: shard of %lld elements, capacity %lld", path,
                          (long long)info.shard_numel, (long long)shard_capacity);
    const uint64_t sbytes = (uint64_t)info.shard_numel * (uint64_t)fsdp::dt_size(info.state_dt);
    if (sbytes > 0 && (!master || !exp_avg || !exp_avg_sq))
        return fsdp::fail(FSDP_E_INVAL, "master, exp_avg and exp_avg_sq must be non-NULL");
    const Piece pieces[3] = {{nullptr, (char*)master, sbytes},
                             {nullptr, (char*)exp_avg, sbytes},
                             {nullptr, (char*)exp_avg_sq, sbytes}};
    const int fd = fileno(in.f);
    uint64_t foff = h.payload_offset;   // read_header bounded the payload by the file's length
    uint32_t crc = 0xFFFFFFFFu;
    if (on_device) {
        Staging st;
        hipError_t e = st.init();
        if (e != hipSuccess) return fsdp::hip_fail(e, "pinned staging allocation");
        hipStream_t s = (hipStream_t)stream;
        size_t k = 0;
        for (const Piece& p : pieces) {
            for (uint64_t off = 0; off < p.bytes; off += kChunk, ++k) {
                const size_t n = (size_t)std::min<uint64_t>(kChunk, p.bytes - off);
                // the staging buffer of chunk k was last used by chunk k-2's copy,
                // which ran while chunk k-1 was read
                if (k >= 2 && (e = hipEventSynchronize(st.ev[k % 2])) != hipSuccess)
                    return fsdp::hip_fail(e, "host-to-device copy");
                if (!read_sum(fd, foff, (char*)st.buf[k % 2], n, crc))
                    return fsdp::fail(FSDP_E_FORMAT, "%s: truncated payload", path);
                foff += n;
                e = hipMemcpyAsync(p.dst + off, st.buf[k % 2], n, hipMemcpyHostToDevice, s);
                if (e == hipSuccess) e = hipEventRecord(st.ev[k % 2], s);
                if (e != hipSuccess) return fsdp::hip_fail(e, "host-to-device copy");
            }
        }
        for (int i = 0; i < 2; ++i)
            if ((e = hipEventSynchronize(st.ev[i])) != hipSuccess) return fsdp::hip_fail(e, "host-to-device copy");
    } else {
        for (const Piece& p : pieces) {
            if (!read_sum(fd, foff, p.dst, (size_t)p.bytes, crc))
                return fsdp::fail(FSDP_E_FORMAT, "%s: truncated payload", path);
            foff += p.bytes;
        }
    }
    if ((crc ^ 0xFFFFFFFFu) != h.crc_payload)
        return fsdp::fail(FSDP_E_FORMAT, "%s: payload checksum mismatch (destination contents unspecified)", path);
    if (info_out) *info_out = info;
    return fsdp::ok();
}

}  // extern "C"
