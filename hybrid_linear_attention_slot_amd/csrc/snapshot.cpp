// State snapshots of one slot on disk (gdn_snapshot.h).
//
// "Kapitsa 源码拆解 05": the disk copy of a slot's recurrent state is written
// to a temporary file with the CRC-32C of its header and payload, renamed into
// place when complete, and checked (identity, header, payload) when read; a
// damaged file can be dropped.  Host code only: device<->host copies on the
// caller's stream, which these calls synchronise.
#include <fcntl.h>
#include <stdint.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <string>
#include <vector>

#include "gdn_internal.h"
#include "gdn_snapshot.h"

using gdn::fail;

namespace {

// ---- CRC-32C (Castagnoli, reflected polynomial 0x82F63B78) ----------------
// Slice-by-8 tables built once; the SSE4.2 crc32 instruction computes the
// same polynomial and is used when the CPU has it.
struct CrcTables {
    uint32_t t[8][256];
    CrcTables()
    {
        for (uint32_t i = 0; i < 256; ++i) {
            uint32_t c = i;
            for (int k = 0; k < 8; ++k)
                c = (c >> 1) ^ (0x82F63B78u & (0u - (c & 1u)));
            t[0][i] = c;
        }
        for (uint32_t i = 0; i < 256; ++i)
            for (int s = 1; s < 8; ++s)
                t[s][i] = (t[s - 1][i] >> 8) ^ t[0][t[s - 1][i] & 0xFFu];
    }
};
const CrcTables& tables()
{
    static const CrcTables tb;
    return tb;
}

uint32_t crc_soft(uint32_t c, const uint8_t* p, size_t n)
{
    const CrcTables& tb = tables();
    while (n >= 8) {
        uint64_t w;
        memcpy(&w, p, 8);
        w ^= c;
        c = tb.t[7][w & 0xFF] ^ tb.t[6][(w >> 8) & 0xFF] ^ tb.t[5][(w >> 16) & 0xFF] ^
            tb.t[4][(w >> 24) & 0xFF] ^ tb.t[3][(w >> 32) & 0xFF] ^ tb.t[2][(w >> 40) & 0xFF] ^
            tb.t[1][(w >> 48) & 0xFF] ^ tb.t[0][w >> 56];
        p += 8;
        n -= 8;
    }
    while (n--)
        c = (c >> 8) ^ tb.t[0][(c ^ *p++) & 0xFFu];
    return c;
}

__attribute__((target("sse4.2"))) uint32_t crc_hw(uint32_t c, const uint8_t* p, size_t n)
{
    uint64_t c64 = c;
    while (n >= 8) {
        uint64_t w;
        memcpy(&w, p, 8);
        c64 = __builtin_ia32_crc32di(c64, w);
        p += 8;
        n -= 8;
    }
    uint32_t c32 = uint32_t(c64);
    while (n--)
        c32 = __builtin_ia32_crc32qi(c32, *p++);
    return c32;
}

// ---- file format ---------------------------------------------------------
constexpr char kMagic[8] = {'G', 'D', 'N', 'S', 'T', 'A', 'T', '1'};
constexpr uint32_t kVersion = 1;
constexpr size_t kHeader = 128;
constexpr size_t kHeaderCrcAt = 100;

template <typename T>
void put(uint8_t* h, size_t off, T v)
{
    memcpy(h + off, &v, sizeof(T));
}
template <typename T>
T get(const uint8_t* h, size_t off)
{
    T v;
    memcpy(&v, h + off, sizeof(T));
    return v;
}

struct Layout {
    int32_t nl, C, W, Hk, Hv, dk, dv;
    int64_t win, st;
};

Layout layout_of(const gdn_pool* p)
{
    const gdn_pool_desc& d = p->desc;
    return Layout{int32_t(p->linear.size()), d.conv_channels, d.conv_width, d.num_k_heads,
                  d.num_v_heads, d.head_k_dim, d.head_v_dim, p->conv_bytes, p->ssm_bytes};
}

void build_header(uint8_t* h, const Layout& L, uint64_t key, int64_t position,
                  int64_t payload_bytes, uint32_t payload_crc)
{
    memset(h, 0, kHeader);
    memcpy(h, kMagic, 8);
    put<uint32_t>(h, 8, kVersion);
    put<uint32_t>(h, 12, uint32_t(kHeader));
    put<uint64_t>(h, 16, key);
    put<int64_t>(h, 24, position);
    const int32_t f[9] = {L.nl, L.C, L.W, L.Hk, L.Hv, L.dk, L.dv, 1, 2};
    for (int i = 0; i < 9; ++i)
        put<int32_t>(h, 32 + 4 * i, f[i]);
    put<int64_t>(h, 72, L.win);
    put<int64_t>(h, 80, L.st);
    put<int64_t>(h, 88, payload_bytes);
    put<uint32_t>(h, 96, payload_crc);
    put<uint32_t>(h, kHeaderCrcAt, gdn_crc32c(0, h, kHeaderCrcAt));
}

// An open snapshot file whose header has been read and checked.
struct File {
    int fd = -1;
    uint8_t h[kHeader];
    int64_t payload = 0; // bytes after the header, as the header states
    ~File()
    {
        if (fd >= 0)
            close(fd);
    }
};

bool read_all(int fd, uint8_t* p, size_t n, off_t at)
{
    while (n > 0) {
        const ssize_t r = pread(fd, p, n, at);
        if (r <= 0)
            return false;
        p += r;
        n -= size_t(r);
        at += r;
    }
    return true;
}

// Opens `path` and checks its identity, its header checksum and that its size
// is the header's plus the payload the header states (nothing is allocated
// before that); GDN_OK, GDN_EIO or GDN_ECORRUPT.
int open_checked(const char* path, File& f)
{
    f.fd = open(path, O_RDONLY);
    if (f.fd < 0)
        return fail(GDN_EIO, "snapshot: cannot open %s", path);
    struct stat st;
    if (fstat(f.fd, &st) != 0)
        return fail(GDN_EIO, "snapshot: cannot stat %s", path);
    if (uint64_t(st.st_size) < kHeader)
        return fail(GDN_ECORRUPT, "snapshot: %s is shorter than a header", path);
    if (!read_all(f.fd, f.h, kHeader, 0))
        return fail(GDN_EIO, "snapshot: read error on %s", path);
    const uint8_t* h = f.h;
    if (memcmp(h, kMagic, 8) != 0 || get<uint32_t>(h, 8) != kVersion ||
        get<uint32_t>(h, 12) != kHeader)
        return fail(GDN_ECORRUPT, "snapshot: %s is not a version-%u state snapshot", path,
                    kVersion);
    if (get<uint32_t>(h, kHeaderCrcAt) != gdn_crc32c(0, h, kHeaderCrcAt))
        return fail(GDN_ECORRUPT, "snapshot: header checksum mismatch in %s", path);
    f.payload = get<int64_t>(h, 88);
    if (f.payload < 0 || uint64_t(f.payload) != uint64_t(st.st_size) - kHeader)
        return fail(GDN_ECORRUPT, "snapshot: %s is truncated or has trailing bytes", path);
    return GDN_OK;
}

// Reads the payload of a checked file and verifies its checksum.
int read_payload(const char* path, const File& f, std::vector<uint8_t>& buf)
{
    buf.resize(size_t(f.payload));
    if (!read_all(f.fd, buf.data(), buf.size(), off_t(kHeader)))
        return fail(GDN_EIO, "snapshot: read error on %s", path);
    if (get<uint32_t>(f.h, 96) != gdn_crc32c(0, buf.data(), buf.size()))
        return fail(GDN_ECORRUPT, "snapshot: payload checksum mismatch in %s", path);
    return GDN_OK;
}

int hip_fail(const char* what, hipError_t e)
{
    return fail(GDN_EHIP, "snapshot: %s: %s", what, hipGetErrorString(e));
}

int save(const gdn_pool* pool, int32_t slot, uint64_t key, int64_t position, const char* path,
         gdn_stream_t stream)
{
    const Layout L = layout_of(pool);
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t per = L.win + L.st;
    std::vector<uint8_t> buf(kHeader + size_t(per * L.nl));
    for (int32_t i = 0; i < L.nl; ++i) {
        const uint8_t* page = static_cast<const uint8_t*>(pool->bases[pool->linear[i]]) +
                              int64_t(slot) * pool->desc.page_stride_bytes;
        uint8_t* dst = buf.data() + kHeader + i * per;
        hipError_t e = hipMemcpyAsync(dst, page + pool->desc.conv_offset_bytes, size_t(L.win),
                                      hipMemcpyDeviceToHost, s);
        if (e == hipSuccess && L.st > 0)
            e = hipMemcpyAsync(dst + L.win, page + pool->desc.ssm_offset_bytes, size_t(L.st),
                               hipMemcpyDeviceToHost, s);
        if (e != hipSuccess)
            return hip_fail("device-to-host copy", e);
    }
    const hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return hip_fail("synchronise", e);
    const int64_t payload = per * L.nl;
    build_header(buf.data(), L, key, position, payload,
                 gdn_crc32c(0, buf.data() + kHeader, size_t(payload)));
    const std::string tmp = std::string(path) + ".tmp";
    const int fd = open(tmp.c_str(), O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (fd < 0)
        return fail(GDN_EIO, "snapshot: cannot create %s", tmp.c_str());
    size_t done = 0;
    bool ok = true;
    while (done < buf.size()) {
        const ssize_t w = write(fd, buf.data() + done, buf.size() - done);
        if (w <= 0) {
            ok = false;
            break;
        }
        done += size_t(w);
    }
    ok = ok && fsync(fd) == 0;
    ok = (close(fd) == 0) && ok;
    if (!ok || rename(tmp.c_str(), path) != 0) {
        unlink(tmp.c_str());
        return fail(GDN_EIO, "snapshot: cannot write %s", path);
    }
    // make the rename itself durable: sync the directory that holds the file
    const std::string p(path);
    const size_t slash = p.rfind('/');
    const std::string dir = slash == std::string::npos ? "." : (slash == 0 ? "/" : p.substr(0, slash));
    const int dfd = open(dir.c_str(), O_RDONLY | O_DIRECTORY);
    const bool synced = dfd >= 0 && fsync(dfd) == 0;
    if (dfd >= 0)
        close(dfd);
    if (!synced)
        return fail(GDN_EIO, "snapshot: %s written, but its directory could not be synced", path);
    return GDN_OK;
}

int load(const gdn_pool* pool, int32_t slot, const char* path, uint64_t key, int64_t* position,
         gdn_stream_t stream)
{
    File f;
    int rc = open_checked(path, f);
    if (rc != GDN_OK)
        return rc;
    const uint8_t* h = f.h;
    const Layout L = layout_of(pool);
    const int32_t want[9] = {L.nl, L.C, L.W, L.Hk, L.Hv, L.dk, L.dv, 1, 2};
    for (int i = 0; i < 9; ++i)
        if (get<int32_t>(h, 32 + 4 * i) != want[i])
            return fail(GDN_EINVAL, "snapshot: %s has another state layout than the pool", path);
    if (get<int64_t>(h, 72) != L.win || get<int64_t>(h, 80) != L.st)
        return fail(GDN_EINVAL, "snapshot: %s has other region sizes than the pool", path);
    if (get<uint64_t>(h, 16) != key)
        return fail(GDN_EINVAL, "snapshot: %s holds another key", path);
    const int64_t per = L.win + L.st;
    if (f.payload != per * L.nl)
        return fail(GDN_ECORRUPT, "snapshot: %s states a payload of %lld bytes for this layout",
                    path, (long long)f.payload);
    std::vector<uint8_t> buf;
    rc = read_payload(path, f, buf);
    if (rc != GDN_OK)
        return rc;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < L.nl; ++i) {
        uint8_t* page = static_cast<uint8_t*>(pool->bases[pool->linear[i]]) +
                        int64_t(slot) * pool->desc.page_stride_bytes;
        const uint8_t* src = buf.data() + i * per; // buf holds the payload only
        hipError_t e = hipMemcpyAsync(page + pool->desc.conv_offset_bytes, src, size_t(L.win),
                                      hipMemcpyHostToDevice, s);
        if (e == hipSuccess && L.st > 0)
            e = hipMemcpyAsync(page + pool->desc.ssm_offset_bytes, src + L.win, size_t(L.st),
                               hipMemcpyHostToDevice, s);
        if (e != hipSuccess)
            return hip_fail("host-to-device copy", e);
    }
    const hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return hip_fail("synchronise", e);
    *position = get<int64_t>(h, 24);
    return GDN_OK;
}

int read_info(const char* path, gdn_snapshot_info* out)
{
    File f;
    int rc = open_checked(path, f);
    if (rc != GDN_OK)
        return rc;
    std::vector<uint8_t> buf;
    rc = read_payload(path, f, buf);
    if (rc != GDN_OK)
        return rc;
    const uint8_t* h = f.h;
    out->key = get<uint64_t>(h, 16);
    out->position = get<int64_t>(h, 24);
    out->num_linear_layers = get<int32_t>(h, 32);
    out->conv_channels = get<int32_t>(h, 36);
    out->conv_width = get<int32_t>(h, 40);
    out->num_k_heads = get<int32_t>(h, 44);
    out->num_v_heads = get<int32_t>(h, 48);
    out->head_k_dim = get<int32_t>(h, 52);
    out->head_v_dim = get<int32_t>(h, 56);
    out->window_bytes = get<int64_t>(h, 72);
    out->state_bytes = get<int64_t>(h, 80);
    out->payload_bytes = get<int64_t>(h, 88);
    out->payload_crc = get<uint32_t>(h, 96);
    return GDN_OK;
}

} // namespace

extern "C" {

uint32_t gdn_crc32c(uint32_t crc, const void* data, size_t len)
{
    static const bool hw = __builtin_cpu_supports("sse4.2");
    const uint8_t* p = static_cast<const uint8_t*>(data);
    const uint32_t c = ~crc;
    return ~(hw ? crc_hw(c, p, len) : crc_soft(c, p, len));
}

int gdn_snapshot_save(const gdn_pool* pool, int32_t slot, uint64_t key, int64_t position,
                      const char* path, gdn_stream_t stream)
{
    gdn::clear_error();
    if (!pool || !path)
        return fail(GDN_EINVAL, "snapshot: NULL pool or path");
    if (slot < 0 || slot >= pool->desc.num_slots)
        return fail(GDN_ERANGE, "snapshot: slot %d out of range", slot);
    return gdn::guarded([&] { return save(pool, slot, key, position, path, stream); });
}

int gdn_snapshot_load(const gdn_pool* pool, int32_t slot, const char* path, uint64_t key,
                      int64_t* position, int32_t drop_damaged, gdn_stream_t stream)
{
    gdn::clear_error();
    if (!pool || !path || !position)
        return fail(GDN_EINVAL, "snapshot: NULL argument");
    if (slot < 0 || slot >= pool->desc.num_slots)
        return fail(GDN_ERANGE, "snapshot: slot %d out of range", slot);
    return gdn::guarded([&] {
        const int rc = load(pool, slot, path, key, position, stream);
        if (rc == GDN_ECORRUPT && drop_damaged) {
            char msg[512];
            snprintf(msg, sizeof msg, "%s", gdn_last_error());
            unlink(path);
            return fail(GDN_ECORRUPT, "%s (file dropped)", msg);
        }
        return rc;
    });
}

int gdn_snapshot_read_info(const char* path, gdn_snapshot_info* out)
{
    gdn::clear_error();
    if (!path || !out)
        return fail(GDN_EINVAL, "snapshot: NULL argument");
    return gdn::guarded([&] { return read_info(path, out); });
}

} // extern "C"
