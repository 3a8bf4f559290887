// Shard checkpoints: each rank writes its own shard state to its own file
// (a sharded state dict), and a checkpoint taken at D ranks can be loaded
// back at the same D or re-sharded to any D2 on load, each new rank reading
// only the byte ranges it owns from the old files.
//
// File layout (little-endian):
//   [0, 4096)   header: magic "ZSSHARD1", version, rank, D, N, S, step,
//               block size, four array records (p, m, v, w), and a CRC-32C
//               of the header's first 4092 bytes at offset 4092
//   data        p, m, v (fp32) and w (bf16), S elements each, every array at
//               a 4096-aligned offset
//   crc tables  one CRC-32C per block of each array (the last block may be
//               short), so that a partial read verifies exactly the blocks
//               it touches
// The file is written under a temporary name and renamed into place only
// once complete. Data moves through a pinned host staging buffer; these
// calls synchronize the caller's stream, unlike the kernel entry points.

#include <fcntl.h>
#include <unistd.h>

#include <cerrno>
#include <cstddef>
#include <cstring>
#include <string>
#include <vector>

#include "zs_internal.h"

#define ZS_EXPORT extern "C" __attribute__((visibility("default")))

using namespace zs;

namespace {

constexpr char kMagic[8] = {'Z', 'S', 'S', 'H', 'A', 'R', 'D', '1'};
constexpr uint32_t kVersion = 1;
constexpr int64_t kHeaderBytes = 4096;
constexpr int64_t kBlock = int64_t(16) << 20;    // bytes per CRC block
constexpr int64_t kStaging = int64_t(64) << 20;  // pinned staging, a multiple of kBlock
constexpr int kArrays = 4;

struct ArrayRec {
    char name[8];
    int32_t dtype;
    uint32_t reserved;
    uint64_t data_offset;
    uint64_t nbytes;
    uint64_t crc_offset;
    uint64_t n_blocks;
};

struct Header {
    char magic[8];
    uint32_t version;
    uint32_t header_bytes;
    int32_t rank;
    int32_t D;
    int64_t N;
    int64_t S;
    int64_t step;
    int64_t block_bytes;
    ArrayRec arrays[kArrays];
};
static_assert(sizeof(Header) < kHeaderBytes - 4, "header fits its page");
static_assert(sizeof(ArrayRec) == 48 && offsetof(Header, arrays) == 56 &&
                  offsetof(Header, block_bytes) == 48 && offsetof(Header, N) == 24,
              "field offsets of the documented file format");

// CRC-32C (Castagnoli, reflected polynomial 0x82F63B78), initial value and
// final xor 0xFFFFFFFF, computed with the SSE4.2 crc32 instruction.
__attribute__((target("sse4.2"))) uint32_t crc32c(const void* data, size_t n, uint32_t crc = 0) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    uint64_t c = ~crc & 0xFFFFFFFFu;
    while (n >= 8) {
        uint64_t w;
        std::memcpy(&w, p, 8);
        c = __builtin_ia32_crc32di(c, w);
        p += 8;
        n -= 8;
    }
    uint32_t c32 = uint32_t(c);
    while (n--) c32 = __builtin_ia32_crc32qi(c32, *p++);
    return ~c32;
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Fd {
    int fd = -1;
    ~Fd() {
        if (fd >= 0) ::close(fd);
    }
};

// Removes a partly written file unless the save completed.
struct TmpFile {
    std::string path;
    bool keep = false;
    ~TmpFile() {
        if (!keep && !path.empty()) ::unlink(path.c_str());
    }
};

struct Pinned {
    void* p = nullptr;
    ~Pinned() {
        if (p) (void)hipHostFree(p);
    }
};

bool write_all(int fd, const void* buf, int64_t n, int64_t off) {
    const char* b = static_cast<const char*>(buf);
    while (n > 0) {
        const ssize_t w = ::pwrite(fd, b, size_t(n), off);
        if (w < 0 && errno == EINTR) continue;
        if (w <= 0) return false;
        b += w;
        n -= w;
        off += w;
    }
    return true;
}

bool read_all(int fd, void* buf, int64_t n, int64_t off) {
    char* b = static_cast<char*>(buf);
    while (n > 0) {
        const ssize_t r = ::pread(fd, b, size_t(n), off);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        b += r;
        n -= r;
        off += r;
    }
    return true;
}

// Reads and checks a header; fills hdr.
zs_status read_header(int fd, const char* path, Header* hdr) {
    std::vector<unsigned char> page(kHeaderBytes);
    if (!read_all(fd, page.data(), kHeaderBytes, 0))
        return fail(ZS_EIO, "%s: cannot read the header", path);
    uint32_t stored;
    std::memcpy(&stored, page.data() + kHeaderBytes - 4, 4);
    if (std::memcmp(page.data(), kMagic, 8) != 0) return fail(ZS_EIO, "%s: not a shard file", path);
    if (crc32c(page.data(), kHeaderBytes - 4) != stored)
        return fail(ZS_EIO, "%s: header checksum mismatch", path);
    std::memcpy(hdr, page.data(), sizeof(Header));
    if (hdr->version != kVersion)
        return fail(ZS_EIO, "%s: version %u, expected %u", path, hdr->version, kVersion);
    if (hdr->D < 1 || hdr->D > ZS_MAX_D || hdr->rank < 0 || hdr->rank >= hdr->D || hdr->N < 0 ||
        hdr->S != hdr->N / hdr->D + (hdr->N % hdr->D != 0 ? 1 : 0) || hdr->block_bytes != kBlock)
        return fail(ZS_EIO, "%s: inconsistent header", path);
    const int es[kArrays] = {4, 4, 4, 2};
    for (int a = 0; a < kArrays; ++a)
        if (hdr->arrays[a].nbytes != uint64_t(hdr->S) * uint64_t(es[a]) ||
            hdr->arrays[a].n_blocks != uint64_t((int64_t(hdr->arrays[a].nbytes) + kBlock - 1) / kBlock))
            return fail(ZS_EIO, "%s: inconsistent array record %d", path, a);
    return ZS_OK;
}

// Reads bytes [lo, hi) of array a of an open shard file into dst, verifying
// the CRC of every block it touches (whole blocks are read into staging).
zs_status read_range(int fd, const char* path, const Header& h, int a, int64_t lo, int64_t hi,
                     char* staging, std::vector<uint32_t>& crcs, char* dev_dst,
                     hipStream_t stream) {
    const ArrayRec& rec = h.arrays[a];
    if (crcs.size() != rec.n_blocks) {
        crcs.resize(rec.n_blocks);
        if (!read_all(fd, crcs.data(), int64_t(rec.n_blocks) * 4, int64_t(rec.crc_offset)))
            return fail(ZS_EIO, "%s: cannot read the checksum table", path);
    }
    int64_t pos = lo;
    while (pos < hi) {
        // a window of whole blocks starting at pos's block, at most kStaging bytes
        const int64_t win_lo = pos / kBlock * kBlock;
        int64_t win_hi = win_lo + kStaging;
        if (win_hi > round_up(hi, kBlock)) win_hi = round_up(hi, kBlock);
        if (win_hi > int64_t(rec.nbytes)) win_hi = int64_t(rec.nbytes);
        if (!read_all(fd, staging, win_hi - win_lo, int64_t(rec.data_offset) + win_lo))
            return fail(ZS_EIO, "%s: short read of array %d", path, a);
        for (int64_t o = win_lo; o < win_hi; o += kBlock) {
            const int64_t n = win_hi - o < kBlock ? win_hi - o : kBlock;
            if (crc32c(staging + (o - win_lo), size_t(n)) != crcs[size_t(o / kBlock)])
                return fail(ZS_EIO, "%s: checksum mismatch in array %d block %lld", path, a,
                            (long long)(o / kBlock));
        }
        const int64_t take_hi = hi < win_hi ? hi : win_hi;
        hipError_t e = hipMemcpyAsync(dev_dst + (pos - lo), staging + (pos - win_lo),
                                      size_t(take_hi - pos), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_status(e, "zs_shard load copy");
        pos = take_hi;
    }
    return ZS_OK;
}

zs_status check_state_ptrs(const char* who, const float* p, const float* m, const float* v,
                           const uint16_t* w, int64_t S) {
    if (S == 0) return ZS_OK;
    if (!p || !m || !v || !w) return fail(ZS_EINVAL, "%s: p, m, v or w is NULL", who);
    if (!aligned(p, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(w, 2))
        return fail(ZS_EINVAL, "%s: p, m, v or w misaligned", who);
    const Range rs[4] = {range_of(p, S, 4), range_of(m, S, 4), range_of(v, S, 4), range_of(w, S, 2)};
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlap(rs[a], rs[b])) return fail(ZS_EALIAS, "%s: state arrays overlap", who);
    return ZS_OK;
}

}  // namespace

ZS_EXPORT zs_status zs_shard_save(const char* path, const zs_shard_info* info, const float* p,
                                  const float* m, const float* v, const uint16_t* w,
                                  hipStream_t stream) {
    const char* who = "zs_shard_save";
    if (!path || !info) return fail(ZS_EINVAL, "%s: path or info is NULL", who);
    if (info->D < 1 || info->D > ZS_MAX_D || info->rank < 0 || info->rank >= info->D)
        return fail(ZS_EINVAL, "%s: rank %d of D = %d", who, info->rank, info->D);
    if (info->N < 0 || info->N > INT64_MAX / 64)
        return fail(ZS_EINVAL, "%s: N = %lld out of range", who, (long long)info->N);
    const int64_t S = info->N / info->D + (info->N % info->D != 0 ? 1 : 0);
    if (info->S != S)
        return fail(ZS_EINVAL, "%s: S = %lld but ceil(N/D) = %lld", who, (long long)info->S,
                    (long long)S);
    if (info->step < 0) return fail(ZS_EINVAL, "%s: step < 0", who);
    zs_status st = check_state_ptrs(who, p, m, v, w, S);
    if (st != ZS_OK) return st;

    Header h;
    std::memset(&h, 0, sizeof h);
    std::memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.header_bytes = uint32_t(kHeaderBytes);
    h.rank = info->rank;
    h.D = info->D;
    h.N = info->N;
    h.S = S;
    h.step = info->step;
    h.block_bytes = kBlock;
    const char* names[kArrays] = {"p", "m", "v", "w"};
    const void* src[kArrays] = {p, m, v, w};
    const int es[kArrays] = {4, 4, 4, 2};
    int64_t off = kHeaderBytes;
    for (int a = 0; a < kArrays; ++a) {
        ArrayRec& r = h.arrays[a];
        std::strncpy(r.name, names[a], sizeof r.name - 1);
        r.dtype = es[a] == 4 ? ZS_F32 : ZS_BF16;
        r.data_offset = uint64_t(off);
        r.nbytes = uint64_t(S) * uint64_t(es[a]);
        r.n_blocks = (r.nbytes + uint64_t(kBlock) - 1) / uint64_t(kBlock);
        off = round_up(off + int64_t(r.nbytes), 4096);
    }
    for (int a = 0; a < kArrays; ++a) {
        h.arrays[a].crc_offset = uint64_t(off);
        off += int64_t(h.arrays[a].n_blocks) * 4;
    }

    const std::string tmp = std::string(path) + ".tmp";
    Fd f;
    f.fd = ::open(tmp.c_str(), O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (f.fd < 0) return fail(ZS_EIO, "%s: cannot create %s: %s", who, tmp.c_str(), std::strerror(errno));
    TmpFile guard{tmp};
    Pinned stage;
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess && S > 0) e = hipHostMalloc(&stage.p, size_t(kStaging), hipHostMallocDefault);
    if (e != hipSuccess) return hip_status(e, "zs_shard_save: staging");
    char* buf = static_cast<char*>(stage.p);
    for (int a = 0; a < kArrays; ++a) {
        const ArrayRec& r = h.arrays[a];
        std::vector<uint32_t> crcs(r.n_blocks);
        for (int64_t o = 0; o < int64_t(r.nbytes); o += kStaging) {
            const int64_t n = int64_t(r.nbytes) - o < kStaging ? int64_t(r.nbytes) - o : kStaging;
            e = hipMemcpyAsync(buf, static_cast<const char*>(src[a]) + o, size_t(n),
                               hipMemcpyDeviceToHost, stream);
            if (e == hipSuccess) e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_status(e, "zs_shard_save copy");
            for (int64_t b = 0; b < n; b += kBlock) {
                const int64_t bn = n - b < kBlock ? n - b : kBlock;
                crcs[size_t((o + b) / kBlock)] = crc32c(buf + b, size_t(bn));
            }
            if (!write_all(f.fd, buf, n, int64_t(r.data_offset) + o))
                return fail(ZS_EIO, "%s: write failed: %s", who, std::strerror(errno));
        }
        if (!write_all(f.fd, crcs.data(), int64_t(crcs.size()) * 4, int64_t(r.crc_offset)))
            return fail(ZS_EIO, "%s: write failed: %s", who, std::strerror(errno));
    }
    std::vector<unsigned char> page(kHeaderBytes, 0);
    std::memcpy(page.data(), &h, sizeof h);
    const uint32_t hc = crc32c(page.data(), kHeaderBytes - 4);
    std::memcpy(page.data() + kHeaderBytes - 4, &hc, 4);
    if (!write_all(f.fd, page.data(), kHeaderBytes, 0) || ::fsync(f.fd) != 0)
        return fail(ZS_EIO, "%s: write failed: %s", who, std::strerror(errno));
    ::close(f.fd);
    f.fd = -1;
    if (::rename(tmp.c_str(), path) != 0)
        return fail(ZS_EIO, "%s: cannot rename into %s: %s", who, path, std::strerror(errno));
    guard.keep = true;
    return ok();
}

ZS_EXPORT zs_status zs_shard_info_read(const char* path, zs_shard_info* info) {
    if (!path || !info) return fail(ZS_EINVAL, "zs_shard_info_read: path or info is NULL");
    Fd f;
    f.fd = ::open(path, O_RDONLY);
    if (f.fd < 0) return fail(ZS_EIO, "%s: cannot open: %s", path, std::strerror(errno));
    Header h;
    const zs_status st = read_header(f.fd, path, &h);
    if (st != ZS_OK) return st;
    info->rank = h.rank;
    info->D = h.D;
    info->N = h.N;
    info->S = h.S;
    info->step = h.step;
    return ok();
}

ZS_EXPORT zs_status zs_shard_load_resharded(const char* const* paths, int32_t D, int32_t rank,
                                            int32_t D2, float* p, float* m, float* v,
                                            uint16_t* w, int64_t S2, zs_shard_info* info_out,
                                            hipStream_t stream) {
    const char* who = "zs_shard_load_resharded";
    if (!paths) return fail(ZS_EINVAL, "%s: paths is NULL", who);
    if (D < 1 || D > ZS_MAX_D || D2 < 1 || D2 > ZS_MAX_D || rank < 0 || rank >= D2)
        return fail(ZS_EINVAL, "%s: D = %d, rank %d of D2 = %d", who, D, rank, D2);
    std::vector<Fd> fds(static_cast<size_t>(D));
    std::vector<Header> hs(static_cast<size_t>(D));
    for (int r = 0; r < D; ++r) {
        if (!paths[r]) return fail(ZS_EINVAL, "%s: paths[%d] is NULL", who, r);
        fds[r].fd = ::open(paths[r], O_RDONLY);
        if (fds[r].fd < 0)
            return fail(ZS_EIO, "%s: cannot open: %s", paths[r], std::strerror(errno));
        const zs_status st = read_header(fds[r].fd, paths[r], &hs[r]);
        if (st != ZS_OK) return st;
        if (hs[r].D != D || hs[r].rank != r || hs[r].N != hs[0].N || hs[r].step != hs[0].step)
            return fail(ZS_EIO, "%s: file %d holds rank %d of D = %d (step %lld); expected rank %d "
                        "of D = %d from one checkpoint", who, r, hs[r].rank, hs[r].D,
                        (long long)hs[r].step, r, D);
    }
    const int64_t N = hs[0].N, S = hs[0].S;
    const int64_t want_S2 = N / D2 + (N % D2 != 0 ? 1 : 0);
    if (S2 != want_S2)
        return fail(ZS_EINVAL, "%s: S2 = %lld but ceil(N/D2) = %lld", who, (long long)S2,
                    (long long)want_S2);
    zs_status st = check_state_ptrs(who, p, m, v, w, S2);
    if (st != ZS_OK) return st;
    Pinned stage;
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess && S2 > 0) e = hipHostMalloc(&stage.p, size_t(kStaging), hipHostMallocDefault);
    if (e != hipSuccess) return hip_status(e, "zs_shard_load_resharded: staging");
    char* dst[kArrays] = {reinterpret_cast<char*>(p), reinterpret_cast<char*>(m),
                          reinterpret_cast<char*>(v), reinterpret_cast<char*>(w)};
    const int es[kArrays] = {4, 4, 4, 2};
    const int64_t lo = int64_t(rank) * S2;
    const int64_t real_hi = lo + S2 < N ? lo + S2 : N;
    for (int a = 0; a < kArrays; ++a) {
        std::vector<std::vector<uint32_t>> crcs(static_cast<size_t>(D));
        for (int64_t i = lo; i < real_hi;) {
            const int64_t r = i / S;
            const int64_t end = (r + 1) * S < real_hi ? (r + 1) * S : real_hi;
            st = read_range(fds[r].fd, paths[r], hs[r], a, (i - r * S) * es[a], (end - r * S) * es[a],
                            static_cast<char*>(stage.p), crcs[size_t(r)],
                            dst[a] + (i - lo) * es[a], stream);
            if (st != ZS_OK) return st;
            i = end;
        }
        const int64_t pad0 = real_hi > lo ? real_hi - lo : 0;
        if (pad0 < S2) {
            e = hipMemsetAsync(dst[a] + pad0 * es[a], 0, size_t(S2 - pad0) * size_t(es[a]), stream);
            if (e == hipSuccess) e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_status(e, "zs_shard_load_resharded: pad");
        }
    }
    if (info_out) {
        info_out->rank = rank;
        info_out->D = D2;
        info_out->N = N;
        info_out->S = S2;
        info_out->step = hs[0].step;
    }
    return ok();
}

ZS_EXPORT zs_status zs_shard_load(const char* path, float* p, float* m, float* v, uint16_t* w,
                                  int64_t S, zs_shard_info* info_out, hipStream_t stream) {
    if (!path) return fail(ZS_EINVAL, "zs_shard_load: path is NULL");
    zs_shard_info info;
    zs_status st = zs_shard_info_read(path, &info);
    if (st != ZS_OK) return st;
    if (info.S != S)
        return fail(ZS_EINVAL, "zs_shard_load: the file holds S = %lld, the buffers S = %lld",
                    (long long)info.S, (long long)S);
    Fd f;
    f.fd = ::open(path, O_RDONLY);
    if (f.fd < 0) return fail(ZS_EIO, "%s: cannot open: %s", path, std::strerror(errno));
    Header h;
    st = read_header(f.fd, path, &h);
    if (st != ZS_OK) return st;
    st = check_state_ptrs("zs_shard_load", p, m, v, w, S);
    if (st != ZS_OK) return st;
    Pinned stage;
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess && S > 0) e = hipHostMalloc(&stage.p, size_t(kStaging), hipHostMallocDefault);
    if (e != hipSuccess) return hip_status(e, "zs_shard_load: staging");
    char* dst[kArrays] = {reinterpret_cast<char*>(p), reinterpret_cast<char*>(m),
                          reinterpret_cast<char*>(v), reinterpret_cast<char*>(w)};
    for (int a = 0; a < kArrays; ++a) {
        std::vector<uint32_t> crcs;
        if (S == 0) break;
        st = read_range(f.fd, path, h, a, 0, int64_t(h.arrays[a].nbytes),
                        static_cast<char*>(stage.p), crcs, dst[a], stream);
        if (st != ZS_OK) return st;
    }
    if (info_out) *info_out = info;
    return ok();
}
