// Register and memory budgets of the compiled kernels, read from the gfx950
// code object the HIP runtime compiler produced for this program (Tiki
// README, "The architecture we want": register and shared-memory budgets are
// visible before launch). The code object is an ELF file whose AMDGPU note
// (type 32) holds the kernels' metadata as a MessagePack map:
// "amdhsa.kernels" is an array with one map per kernel carrying ".name",
// ".vgpr_count", ".agpr_count", ".sgpr_count", ".vgpr_spill_count",
// ".sgpr_spill_count", ".private_segment_fixed_size" (scratch bytes per
// lane) and ".group_segment_fixed_size" (LDS bytes). Only what this library
// compiled is read; a malformed object yields no entries.
#include <cstring>

#include "graph.hpp"

namespace rv {

namespace {

struct Reader {
    const unsigned char* p;
    const unsigned char* end;
    bool ok = true;

    bool need(size_t n) {
        if (!ok || (size_t)(end - p) < n) ok = false;
        return ok;
    }
    uint64_t be(int n) {
        if (!need((size_t)n)) return 0;
        uint64_t v = 0;
        for (int i = 0; i < n; ++i) v = (v << 8) | p[i];
        p += n;
        return v;
    }
    // A string at the cursor (else ok = false).
    std::string str() {
        if (!need(1)) return "";
        const unsigned c = *p++;
        size_t n;
        if ((c & 0xe0) == 0xa0)
            n = c & 0x1f;
        else if (c == 0xd9)
            n = (size_t)be(1);
        else if (c == 0xda)
            n = (size_t)be(2);
        else if (c == 0xdb)
            n = (size_t)be(4);
        else {
            ok = false;
            return "";
        }
        if (!need(n)) return "";
        std::string s((const char*)p, n);
        p += n;
        return s;
    }
    // An integer at the cursor; false (cursor past the value) if it is not one.
    bool integer(int64_t* v) {
        if (!need(1)) return false;
        const unsigned c = *p;
        if (c <= 0x7f) {
            *v = c;
            ++p;
            return true;
        }
        if (c >= 0xe0) {
            *v = (int64_t)(int8_t)c;
            ++p;
            return true;
        }
        if (c >= 0xcc && c <= 0xcf) {
            ++p;
            *v = (int64_t)be(1 << (c - 0xcc));
            return ok;
        }
        if (c >= 0xd0 && c <= 0xd3) {
            ++p;
            const int n = 1 << (c - 0xd0);
            const uint64_t u = be(n);
            *v = n == 8 ? (int64_t)u : (int64_t)(u << (64 - 8 * n)) >> (64 - 8 * n);
            return ok;
        }
        skip();
        return false;
    }
    // Element count of a map or array header at the cursor (-1 if neither).
    int64_t header(bool map) {
        if (!need(1)) return -1;
        const unsigned c = *p;
        if (map && (c & 0xf0) == 0x80) return ++p, c & 0x0f;
        if (!map && (c & 0xf0) == 0x90) return ++p, c & 0x0f;
        if (c == (map ? 0xde : 0xdc)) return ++p, (int64_t)be(2);
        if (c == (map ? 0xdf : 0xdd)) return ++p, (int64_t)be(4);
        return -1;
    }
    void skip(int depth = 0) {
        if (!need(1) || depth > 64) {
            ok = false;
            return;
        }
        const unsigned c = *p;
        if (c <= 0x7f || c >= 0xe0 || c == 0xc0 || c == 0xc2 || c == 0xc3) {
            ++p;
            return;
        }
        if ((c & 0xe0) == 0xa0 || c == 0xd9 || c == 0xda || c == 0xdb) {
            str();
            return;
        }
        if ((c & 0xf0) == 0x80 || c == 0xde || c == 0xdf) {
            const int64_t n = header(true);
            for (int64_t i = 0; i < 2 * n && ok; ++i) skip(depth + 1);
            return;
        }
        if ((c & 0xf0) == 0x90 || c == 0xdc || c == 0xdd) {
            const int64_t n = header(false);
            for (int64_t i = 0; i < n && ok; ++i) skip(depth + 1);
            return;
        }
        ++p;
        switch (c) {
            case 0xc4: p += need(1) ? be(1) : 0; break;  // bin 8/16/32
            case 0xc5: p += need(2) ? be(2) : 0; break;
            case 0xc6: p += need(4) ? be(4) : 0; break;
            case 0xca: be(4); break;  // float 32/64
            case 0xcb: be(8); break;
            case 0xcc: case 0xd0: be(1); break;
            case 0xcd: case 0xd1: be(2); break;
            case 0xce: case 0xd2: be(4); break;
            case 0xcf: case 0xd3: be(8); break;
            default: ok = false;
        }
        if (p > end) ok = false;
    }
};

template <class T>
static bool at(const std::vector<char>& b, size_t off, T* v) {
    if (off + sizeof(T) > b.size()) return false;
    memcpy(v, b.data() + off, sizeof(T));
    return true;
}

static void parse_kernels(Reader& r, std::map<std::string, KernelResources>& out) {
    const int64_t n = r.header(false);
    for (int64_t i = 0; i < n && r.ok; ++i) {
        const int64_t fields = r.header(true);
        if (fields < 0) {
            r.ok = false;
            return;
        }
        std::string name;
        KernelResources k;
        for (int64_t f = 0; f < fields && r.ok; ++f) {
            const std::string key = r.str();
            int64_t v = 0;
            if (key == ".name") {
                name = r.str();
                continue;
            }
            int64_t* dst = key == ".vgpr_count"                   ? &k.vgpr
                           : key == ".agpr_count"                 ? &k.agpr
                           : key == ".sgpr_count"                 ? &k.sgpr
                           : key == ".vgpr_spill_count"           ? &k.vgpr_spill
                           : key == ".sgpr_spill_count"           ? &k.sgpr_spill
                           : key == ".private_segment_fixed_size" ? &k.scratch
                           : key == ".group_segment_fixed_size"   ? &k.lds
                                                                  : nullptr;
            if (!dst) {
                r.skip();
                continue;
            }
            if (r.integer(&v)) *dst = v;
        }
        if (r.ok && !name.empty()) out[name] = k;
    }
}

}  // namespace

std::map<std::string, KernelResources> kernel_resources(const std::vector<char>& code) {
    std::map<std::string, KernelResources> out;
    if (code.size() < 64 || memcmp(code.data(), "\x7f" "ELF", 4) != 0 || code[4] != 2 || code[5] != 1) return out;
    uint64_t shoff = 0;
    uint16_t shentsize = 0, shnum = 0;
    if (!at(code, 0x28, &shoff) || !at(code, 0x3a, &shentsize) || !at(code, 0x3c, &shnum) || shentsize < 64)
        return out;
    for (uint16_t i = 0; i < shnum; ++i) {
        const size_t sh = (size_t)shoff + (size_t)i * shentsize;
        uint32_t type = 0;
        uint64_t off = 0, size = 0;
        if (!at(code, sh + 4, &type) || !at(code, sh + 24, &off) || !at(code, sh + 32, &size)) return out;
        if (type != 7 || off + size > code.size()) continue;  // SHT_NOTE
        size_t q = (size_t)off;
        const size_t qend = (size_t)(off + size);
        while (q + 12 <= qend) {
            uint32_t namesz = 0, descsz = 0, ntype = 0;
            at(code, q, &namesz);
            at(code, q + 4, &descsz);
            at(code, q + 8, &ntype);
            const size_t name_at = q + 12, desc_at = name_at + ((namesz + 3) & ~3u);
            const size_t next = desc_at + ((descsz + 3) & ~3u);
            if (next > qend) break;
            if (ntype == 32 && namesz >= 6 && memcmp(code.data() + name_at, "AMDGPU", 6) == 0) {
                Reader r{(const unsigned char*)code.data() + desc_at, (const unsigned char*)code.data() + desc_at + descsz};
                const int64_t n = r.header(true);
                for (int64_t f = 0; f < n && r.ok; ++f) {
                    const std::string key = r.str();
                    if (key == "amdhsa.kernels")
                        parse_kernels(r, out);
                    else
                        r.skip();
                }
            }
            q = next;
        }
    }
    return out;
}

}  // namespace rv
