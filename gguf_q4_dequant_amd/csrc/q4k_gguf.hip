// GGUF tensor directory (host code only): where the packed Q4_K bytes of a
// checkpoint sit, so that they can be uploaded unchanged.  The pages load
// GGUF checkpoints and keep their K-quant tensors packed (rlx-qwen3 crate
// page, "Quick start"); the container layout itself is not on the pages and
// follows the published GGUF description, versions 2 and 3:
//   "GGUF" magic, u32 version, u64 tensor count, u64 metadata count,
//   metadata pairs (string key, u32 value type, value),
//   tensor infos (string name, u32 dims, u64 dims[], u32 type, u64 offset),
//   padding to general.alignment (32 unless the metadata sets it), data.
// Strings are a u64 length and the bytes; all integers little endian.
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/q4k.h"

namespace {

constexpr uint32_t kTypeF32 = 0, kTypeF16 = 1;
constexpr uint64_t kMaxString = 1u << 20;  // sanity bounds on a malformed file
constexpr uint64_t kMaxArray = 1ull << 32;

struct Reader {
    FILE *f;
    bool ok = true;
    uint64_t pos = 0;
    bool bytes(void *dst, size_t n) {
        if (!ok) return false;
        if (n && fread(dst, 1, n, f) != n) ok = false;
        pos += n;
        return ok;
    }
    bool skip(uint64_t n) {
        if (!ok) return false;
        if (n && fseek(f, static_cast<long>(n), SEEK_CUR) != 0) ok = false;
        pos += n;
        return ok;
    }
    template <class T> T get() {
        unsigned char b[sizeof(T)] = {};
        bytes(b, sizeof(T));
        T v = 0;
        for (size_t i = 0; i < sizeof(T); ++i) v |= static_cast<T>(static_cast<T>(b[i]) << (8 * i));
        return v;
    }
    bool string(std::string *out) {
        const uint64_t n = get<uint64_t>();
        if (!ok || n > kMaxString) return ok = false;
        if (!out) return skip(n);
        out->resize(n);
        return bytes(n ? &(*out)[0] : nullptr, n);
    }
};

// Size of one scalar of a metadata value type, 0 for string/array/unknown.
uint64_t scalar_size(uint32_t t) {
    switch (t) {
    case 0: case 1: case 7: return 1;  // u8, i8, bool
    case 2: case 3: return 2;          // u16, i16
    case 4: case 5: case 6: return 4;  // u32, i32, f32
    case 10: case 11: case 12: return 8;  // u64, i64, f64
    default: return 0;
    }
}

// Skips one metadata value of type t; reads a u32/u64 alignment if asked.
bool skip_value(Reader &r, uint32_t t, uint64_t *as_uint) {
    if (t == 8) return r.string(nullptr);
    if (t == 9) {
        const uint32_t et = r.get<uint32_t>();
        const uint64_t n = r.get<uint64_t>();
        if (!r.ok || n > kMaxArray || et == 9) return false;  // nested arrays are not produced by writers
        if (et == 8) {
            for (uint64_t i = 0; i < n; ++i)
                if (!r.string(nullptr)) return false;
            return true;
        }
        const uint64_t s = scalar_size(et);
        return s && r.skip(s * n);
    }
    const uint64_t s = scalar_size(t);
    if (!s) return false;
    if (as_uint && (t == 4 || t == 10)) {
        *as_uint = t == 4 ? r.get<uint32_t>() : r.get<uint64_t>();
        return r.ok;
    }
    return r.skip(s);
}

}  // namespace

extern "C" int q4k_gguf_list(const char *path, q4k_gguf_tensor *tensors, int capacity, int *count) {
    if (!path || !count || (capacity > 0 && !tensors)) return Q4K_ERR_NULL;
    if (capacity < 0) return Q4K_ERR_BAD_DIM;
    *count = 0;
    FILE *f = fopen(path, "rb");
    if (!f) return Q4K_ERR_IO;
    Reader r{f};
    int rc = Q4K_OK;
    do {
        char magic[4];
        if (!r.bytes(magic, 4) || memcmp(magic, "GGUF", 4) != 0) { rc = Q4K_ERR_FORMAT; break; }
        const uint32_t version = r.get<uint32_t>();
        if (!r.ok || (version != 2 && version != 3)) { rc = Q4K_ERR_FORMAT; break; }
        const uint64_t n_tensors = r.get<uint64_t>();
        const uint64_t n_kv = r.get<uint64_t>();
        if (!r.ok || n_tensors > (1u << 24) || n_kv > (1u << 24)) { rc = Q4K_ERR_FORMAT; break; }
        uint64_t alignment = 32;
        for (uint64_t i = 0; i < n_kv && rc == Q4K_OK; ++i) {
            std::string key;
            if (!r.string(&key)) { rc = Q4K_ERR_FORMAT; break; }
            const uint32_t t = r.get<uint32_t>();
            uint64_t v = 0;
            const bool want = key == "general.alignment";
            if (!skip_value(r, t, want ? &v : nullptr)) { rc = Q4K_ERR_FORMAT; break; }
            if (want) {
                if (v == 0 || (v & (v - 1)) != 0) { rc = Q4K_ERR_FORMAT; break; }  // a power of two
                alignment = v;
            }
        }
        if (rc != Q4K_OK) break;
        std::vector<q4k_gguf_tensor> all;
        for (uint64_t i = 0; i < n_tensors; ++i) {
            q4k_gguf_tensor e;
            memset(&e, 0, sizeof(e));
            std::string name;
            if (!r.string(&name) || name.size() >= sizeof(e.name)) { rc = Q4K_ERR_FORMAT; break; }
            memcpy(e.name, name.data(), name.size());
            e.n_dims = r.get<uint32_t>();
            if (!r.ok || e.n_dims < 1 || e.n_dims > 4) { rc = Q4K_ERR_FORMAT; break; }
            for (int d = 0; d < 4; ++d) e.dims[d] = 1;
            uint64_t elems = 1;
            for (uint32_t d = 0; d < e.n_dims; ++d) {
                e.dims[d] = r.get<uint64_t>();
                if (e.dims[d] == 0 || e.dims[d] > (1ull << 40) || elems > (1ull << 62) / e.dims[d]) {
                    r.ok = false;
                    break;
                }
                elems *= e.dims[d];
            }
            e.type = r.get<uint32_t>();
            e.offset = r.get<uint64_t>();  // relative to the data section for now
            if (!r.ok || e.offset % alignment != 0) { rc = Q4K_ERR_FORMAT; break; }
            if (e.type == Q4K_GGUF_TYPE_Q4_K) {
                if (e.dims[0] % Q4K_BLOCK_WEIGHTS != 0) { rc = Q4K_ERR_FORMAT; break; }
                e.nbytes = elems / Q4K_BLOCK_WEIGHTS * Q4K_BLOCK_BYTES;
            } else if (e.type == kTypeF32) {
                e.nbytes = elems * 4;
            } else if (e.type == kTypeF16) {
                e.nbytes = elems * 2;
            }
            all.push_back(e);
        }
        if (rc != Q4K_OK) break;
        const uint64_t data = (r.pos + alignment - 1) / alignment * alignment;
        if (fseek(f, 0, SEEK_END) != 0) { rc = Q4K_ERR_IO; break; }
        const long end = ftell(f);
        if (end < 0) { rc = Q4K_ERR_IO; break; }
        for (q4k_gguf_tensor &e : all) {
            e.offset += data;
            if (e.offset + e.nbytes > static_cast<uint64_t>(end)) { rc = Q4K_ERR_FORMAT; break; }  // truncated
        }
        if (rc != Q4K_OK) break;
        for (size_t i = 0; i < all.size() && static_cast<int>(i) < capacity; ++i) tensors[i] = all[i];
        *count = static_cast<int>(all.size());
    } while (false);
    if (!r.ok && rc == Q4K_OK) rc = Q4K_ERR_FORMAT;
    fclose(f);
    return rc;
}
