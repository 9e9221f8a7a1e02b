// .smoe vault reader and writer (host code; include/smoe_vault.h is the
// ABI). Layout and rules: ".smoe Binary Format" -- File Architecture, File
// Header, Version acceptance, Arch Block "SARC", Expert Table Entry, Flash
// Lookup, Tensor Descriptor, Expert Blob Architecture.
//
// Files are read and written with pread / pwrite at absolute offsets (every
// offset in the format is from the start of the file). Blobs bound for or
// coming from the GPU pass through pinned staging buffers the handle owns;
// a layer is streamed with two of them so that the disk read of one expert
// overlaps the host-to-device copy of the previous one.

#include <errno.h>
#include <fcntl.h>
#include <hip/hip_runtime.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/smoe_vault.h"
#include "smoe_internal.hpp"

using smoe::report_error;
using smoe::report_ok;

namespace {

constexpr uint8_t kMagic[8] = {0x53, 0x4D, 0x4F, 0x45, 0xDE, 0xEA, 0x00, 0x01};
constexpr uint8_t kSarc[4] = {0x53, 0x41, 0x52, 0x43};
constexpr uint64_t kPage = SMOE_BLOB_ALIGN;
constexpr uint64_t kMetaPerExpert = sizeof(smoe_expert_entry) + 3 * sizeof(smoe_tensor_desc);

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

template <size_t N>
bool all_zero(const uint8_t (&b)[N]) {
  for (size_t i = 0; i < N; ++i)
    if (b[i]) return false;
  return true;
}

uint64_t key_of(uint32_t layer, uint32_t expert) { return ((uint64_t)layer << 32) | expert; }

// The arch block rules of a v2 vault; nullptr when the block is valid.
const char* arch_problem(const smoe_arch_block& a) {
  if (memcmp(a.magic, kSarc, 4) != 0) return "arch block magic is not SARC";
  if (a.block_version != 1) return "arch block_version is not 1";
  if (a.block_size != SMOE_SARC_SIZE) return "arch block_size is not 128";
  if (a.activation != 0) return "activation is not 0 (SiLU)";
  if (a.moe_top_k < 1 || a.moe_top_k > SMOE_MAX_TOP_K) return "moe_top_k outside 1..16";
  if (a.head_dim > 256) return "head_dim above 256";
  if (a.num_kv_heads == 0 || a.num_heads % a.num_kv_heads != 0)
    return "num_kv_heads does not divide num_heads";
  if (!all_zero(a.reserved)) return "arch block reserved bytes are not zero";
  return nullptr;
}

bool read_at(int fd, void* buf, uint64_t n, uint64_t off) {
  uint8_t* p = (uint8_t*)buf;
  while (n) {
    const ssize_t r = pread(fd, p, n > (1u << 30) ? (1u << 30) : n, (off_t)off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return false;
    p += r;
    n -= (uint64_t)r;
    off += (uint64_t)r;
  }
  return true;
}

bool write_at(int fd, const void* buf, uint64_t n, uint64_t off) {
  const uint8_t* p = (const uint8_t*)buf;
  while (n) {
    const ssize_t r = pwrite(fd, p, n > (1u << 30) ? (1u << 30) : n, (off_t)off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return false;
    p += r;
    n -= (uint64_t)r;
    off += (uint64_t)r;
  }
  return true;
}

int hip_fail(hipError_t e, const char* what) {
  return report_error(SMOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Two pinned host buffers and their copy-done events.
struct Staging {
  void* buf[2] = {nullptr, nullptr};
  hipEvent_t done[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  uint64_t cap = 0;

  int ensure(uint64_t n) {
    if (n <= cap) return SMOE_OK;
    release();
    for (int i = 0; i < 2; ++i) {
      hipError_t e = hipHostMalloc(&buf[i], n, hipHostMallocDefault);
      if (e != hipSuccess) return hip_fail(e, "pinned staging allocation");
      e = hipEventCreateWithFlags(&done[i], hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "staging event");
    }
    cap = n;
    return SMOE_OK;
  }
  // Wait until buffer i is no longer read by a copy.
  int wait(int i) {
    if (!pending[i]) return SMOE_OK;
    pending[i] = false;
    const hipError_t e = hipEventSynchronize(done[i]);
    return e == hipSuccess ? SMOE_OK : hip_fail(e, "staging copy");
  }
  int wait_all() {
    const int a = wait(0), b = wait(1);
    return a ? a : b;
  }
  void release() {
    wait_all();
    for (int i = 0; i < 2; ++i) {
      if (buf[i]) (void)hipHostFree(buf[i]);
      if (done[i]) (void)hipEventDestroy(done[i]);
      buf[i] = nullptr;
      done[i] = nullptr;
    }
    cap = 0;
  }
  ~Staging() { release(); }
};

// Metadata of a vault written from a spec.
struct Plan {
  smoe_vault_header h;
  smoe_arch_block arch;
  smoe_expert_layout L;
  std::vector<smoe_expert_entry> entries;
  std::vector<smoe_tensor_desc> descs;
  uint64_t file_size;
};

void fill_descs(const smoe_expert_layout& L, smoe_tensor_desc* d) {
  const smoe_tensor_layout* t[3] = {&L.gate, &L.up, &L.down};
  for (int k = 0; k < 3; ++k) {
    memset(&d[k], 0, sizeof d[k]);
    d[k].tensor_type = (uint8_t)k;
    d[k].ndim = 2;
    d[k].rows = t[k]->rows;
    d[k].cols = t[k]->cols;
    d[k].packed_offset = t[k]->codes_offset;
    d[k].packed_size = t[k]->codes_bytes;
    d[k].scales_offset = t[k]->scales_offset;
    d[k].scales_size = t[k]->scales_bytes;
  }
}

int make_plan(const smoe_vault_spec* s, Plan* p, bool with_tables) {
  if (!s) return report_error(SMOE_E_ARG, "null spec");
  if (s->version != 1 && s->version != 2)
    return report_error(SMOE_E_ARG, "version must be 1 or 2 (got %u)", s->version);
  if (s->num_moe_layers < 1 || s->experts_per_layer < 1)
    return report_error(SMOE_E_ARG, "need at least one layer and one expert per layer");
  if (!s->layer_ids) return report_error(SMOE_E_ARG, "null layer_ids");
  for (uint32_t i = 1; i < s->num_moe_layers; ++i)
    if (s->layer_ids[i] <= s->layer_ids[i - 1])
      return report_error(SMOE_E_ARG, "layer_ids must be strictly ascending");
  int rc = smoe_expert_layout_of(s->d_model, s->moe_ffn_dim, s->bits, SMOE_SCALE_F16, &p->L);
  if (rc) return rc;
  const uint64_t n = (uint64_t)s->num_moe_layers * s->experts_per_layer;
  if (n > 0xFFFFFFFFull) return report_error(SMOE_E_ARG, "more than 2^32-1 experts");
  const uint64_t meta_end = SMOE_VAULT_TABLE_OFFSET + n * kMetaPerExpert;
  memset(&p->arch, 0, sizeof p->arch);
  uint64_t arch_off = 0, end = meta_end;
  if (s->version == 2) {
    if (!s->arch) return report_error(SMOE_E_ARG, "a version 2 vault needs an arch block");
    if (const char* why = arch_problem(*s->arch)) return report_error(SMOE_E_ARG, "%s", why);
    p->arch = *s->arch;
    arch_off = round_up(meta_end, 64);
    end = arch_off + SMOE_SARC_SIZE;
    if (arch_off > 0xFFFFFFFFull)
      return report_error(SMOE_E_ARG, "metadata too large for a 32-bit arch offset");
  } else if (s->arch) {
    return report_error(SMOE_E_ARG, "a version 1 vault has no arch block");
  }
  smoe_vault_header& h = p->h;
  memset(&h, 0, sizeof h);
  memcpy(h.magic, kMagic, 8);
  h.version = s->version;
  h.num_moe_layers = s->num_moe_layers;
  h.max_experts_per_layer = s->experts_per_layer;
  h.total_experts = (uint32_t)n;
  h.table_offset = SMOE_VAULT_TABLE_OFFSET;
  h.data_offset = round_up(end, kPage);
  h.group_size = SMOE_GROUP_SIZE;
  h.bits = s->bits;
  h.d_model = s->d_model;
  h.vocab_size = s->vocab_size;
  h.ffn_dim = s->ffn_dim;
  h.reserved_ext = (uint32_t)arch_off;
  p->file_size = h.data_offset + n * p->L.padded_size;
  if (!with_tables) return SMOE_OK;
  const smoe_expert_layout& L = p->L;
  const uint64_t groups = ceil_div((uint64_t)L.gate.rows * L.gate.cols, SMOE_GROUP_SIZE) +
                          ceil_div((uint64_t)L.up.rows * L.up.cols, SMOE_GROUP_SIZE) +
                          ceil_div((uint64_t)L.down.rows * L.down.cols, SMOE_GROUP_SIZE);
  try {
    p->entries.resize(n);
    p->descs.resize(n * 3);
  } catch (const std::bad_alloc&) {
    return report_error(SMOE_E_ARG, "out of host memory for %llu table entries",
                        (unsigned long long)n);
  }
  for (uint64_t i = 0; i < n; ++i) {
    smoe_expert_entry& e = p->entries[i];
    memset(&e, 0, sizeof e);
    e.layer_id = s->layer_ids[i / s->experts_per_layer];
    e.expert_id = (uint32_t)(i % s->experts_per_layer);
    e.byte_offset = h.data_offset + i * L.padded_size;
    e.raw_size = L.raw_size;
    e.padded_size = L.padded_size;
    e.group_size = SMOE_GROUP_SIZE;
    e.num_groups = groups;
    fill_descs(L, &p->descs[i * 3]);
  }
  return SMOE_OK;
}

}  // namespace

struct smoe_vault_writer {
  int fd = -1;
  Plan plan;
  std::vector<uint32_t> layer_ids;
  std::vector<uint8_t> written;
  Staging st;
};

struct smoe_vault {
  int fd = -1;
  uint64_t size = 0;
  smoe_vault_header h;
  smoe_arch_block arch;
  std::vector<smoe_expert_entry> entries;
  std::vector<smoe_tensor_desc> descs;
  std::unordered_map<uint64_t, uint32_t> index;  // (layer, expert) -> entry
  Staging st;
};

namespace {

// Every reader check of the header, arch block, table and descriptors.
int validate(smoe_vault* v) {
#define BAD(...) return report_error(SMOE_E_FORMAT, __VA_ARGS__)
  const smoe_vault_header& h = v->h;
  if (memcmp(h.magic, kMagic, 8) != 0) BAD("bad magic (not a .smoe vault)");
  if (h.version != 1 && h.version != 2) BAD("unsupported version %u (readers take 1-2)", h.version);
  if (h.table_offset != SMOE_VAULT_TABLE_OFFSET) BAD("table_offset is not 64");
  if (h.group_size != SMOE_GROUP_SIZE) BAD("group_size is not 64");
  if (h.bits != 2 && h.bits != 4) BAD("bits is not 2 or 4");
  if (h.total_experts < 1) BAD("the expert table is empty");
  if (h.data_offset % kPage) BAD("data_offset is not a multiple of 16384");
  const uint64_t n = h.total_experts;
  const uint64_t meta_end = SMOE_VAULT_TABLE_OFFSET + n * kMetaPerExpert;
  if (h.data_offset < meta_end) BAD("data_offset overlaps the table or descriptors");
  if (h.data_offset > v->size) BAD("data_offset past the end of the file");
  memset(&v->arch, 0, sizeof v->arch);
  if (h.version == 1) {
    if (h.reserved_ext != 0) BAD("version 1 vault with a nonzero reserved_ext");
  } else {
    const uint64_t a = h.reserved_ext;
    if (a % 64) BAD("arch block offset is not a multiple of 64");
    if (a < meta_end) BAD("arch block overlaps the table or descriptors");
    if (a + SMOE_SARC_SIZE > h.data_offset) BAD("arch block runs into the expert data");
    if (!read_at(v->fd, &v->arch, sizeof v->arch, a))
      return report_error(SMOE_E_IO, "reading the arch block failed");
    if (const char* why = arch_problem(v->arch)) BAD("%s", why);
  }
  try {
    v->entries.resize(n);
    v->descs.resize(n * 3);
  } catch (const std::bad_alloc&) {
    return report_error(SMOE_E_IO, "out of host memory for the table");
  }
  if (!read_at(v->fd, v->entries.data(), n * sizeof(smoe_expert_entry), SMOE_VAULT_TABLE_OFFSET) ||
      !read_at(v->fd, v->descs.data(), n * 3 * sizeof(smoe_tensor_desc),
               SMOE_VAULT_TABLE_OFFSET + n * sizeof(smoe_expert_entry)))
    return report_error(SMOE_E_IO, "reading the table failed");
  uint32_t layers = 0, max_per = 0, run = 0;
  std::vector<std::pair<uint64_t, uint64_t>> spans(n);
  for (uint64_t i = 0; i < n; ++i) {
    const smoe_expert_entry& e = v->entries[i];
    if (i > 0) {
      const smoe_expert_entry& p = v->entries[i - 1];
      if (key_of(e.layer_id, e.expert_id) <= key_of(p.layer_id, p.expert_id))
        BAD("table entry %llu is not after entry %llu in (layer, expert) order",
            (unsigned long long)i, (unsigned long long)i - 1);
    }
    if (i == 0 || e.layer_id != v->entries[i - 1].layer_id) {
      ++layers;
      run = 0;
    }
    max_per = std::max(max_per, ++run);
    if (e.group_size != h.group_size) BAD("entry %llu: group_size differs from the header", (unsigned long long)i);
    if (!all_zero(e.reserved)) BAD("entry %llu: reserved bytes are not zero", (unsigned long long)i);
    if (e.byte_offset % kPage) BAD("entry %llu: blob offset is not 16 KB aligned", (unsigned long long)i);
    if (e.byte_offset < h.data_offset) BAD("entry %llu: blob before data_offset", (unsigned long long)i);
    if (e.raw_size > (1ull << 48) || e.padded_size != round_up(e.raw_size, kPage))
      BAD("entry %llu: padded_size is not raw_size rounded up to 16 KB", (unsigned long long)i);
    if (e.byte_offset > v->size || e.padded_size > v->size - e.byte_offset)
      BAD("entry %llu: blob runs past the end of the file", (unsigned long long)i);
    spans[i] = {e.byte_offset, e.padded_size};
    // descriptors
    const smoe_tensor_desc* d = &v->descs[i * 3];
    uint64_t groups = 0;
    std::pair<uint64_t, uint64_t> r[6];
    for (int k = 0; k < 3; ++k) {
      if (d[k].tensor_type != k) BAD("entry %llu: descriptor %d has tensor_type %u", (unsigned long long)i, k, d[k].tensor_type);
      if (d[k].ndim != 2) BAD("entry %llu: descriptor %d is not 2-D", (unsigned long long)i, k);
      if (d[k].reserved_0[0] || d[k].reserved_0[1]) BAD("entry %llu: descriptor %d reserved bytes are not zero", (unsigned long long)i, k);
      const uint64_t cnt = (uint64_t)d[k].rows * d[k].cols;
      if (cnt > (1ull << 48))  // keeps the size arithmetic below exact
        BAD("entry %llu: descriptor %d shape is implausibly large", (unsigned long long)i, k);
      if (d[k].packed_size != ceil_div(cnt * h.bits, 8))
        BAD("entry %llu: descriptor %d packed_size is not ceil(rows*cols*bits/8)", (unsigned long long)i, k);
      if (d[k].scales_size != ceil_div(cnt, SMOE_GROUP_SIZE) * 2)
        BAD("entry %llu: descriptor %d scales_size is not ceil(rows*cols/64)*2", (unsigned long long)i, k);
      groups += ceil_div(cnt, SMOE_GROUP_SIZE);
      r[2 * k] = {d[k].packed_offset, d[k].packed_size};
      r[2 * k + 1] = {d[k].scales_offset, d[k].scales_size};
    }
    const uint32_t ffn = d[0].rows;
    if (ffn < 1 || d[1].rows != ffn || d[2].cols != ffn || d[0].cols != h.d_model ||
        d[1].cols != h.d_model || d[2].rows != h.d_model)
      BAD("entry %llu: shapes are not gate/up [ffn, d_model], down [d_model, ffn]", (unsigned long long)i);
    if (e.num_groups != groups) BAD("entry %llu: num_groups does not match the descriptors", (unsigned long long)i);
    std::sort(r, r + 6);
    for (int k = 0; k < 6; ++k) {
      if (r[k].first > e.raw_size || r[k].second > e.raw_size - r[k].first)
        BAD("entry %llu: a tensor range runs past raw_size", (unsigned long long)i);
      if (k > 0 && r[k].first < r[k - 1].first + r[k - 1].second)
        BAD("entry %llu: tensor ranges overlap", (unsigned long long)i);
    }
  }
  if (layers != h.num_moe_layers) BAD("num_moe_layers is %u, the table has %u layers", h.num_moe_layers, layers);
  if (max_per != h.max_experts_per_layer)
    BAD("max_experts_per_layer is %u, the largest layer has %u", h.max_experts_per_layer, max_per);
  std::sort(spans.begin(), spans.end());
  for (uint64_t i = 1; i < n; ++i)
    if (spans[i].first < spans[i - 1].first + spans[i - 1].second) BAD("expert blobs overlap");
  try {
    v->index.reserve(n);
    for (uint64_t i = 0; i < n; ++i)
      v->index.emplace(key_of(v->entries[i].layer_id, v->entries[i].expert_id), (uint32_t)i);
  } catch (const std::bad_alloc&) {
    return report_error(SMOE_E_IO, "out of host memory for the lookup");
  }
  return SMOE_OK;
#undef BAD
}

// Canonical layout of entry i's shape (fp16 scales).
int canonical(const smoe_vault* v, uint32_t i, smoe_expert_layout* L) {
  const smoe_tensor_desc* d = &v->descs[(uint64_t)i * 3];
  if (smoe_expert_layout_of(v->h.d_model, d[0].rows, v->h.bits, SMOE_SCALE_F16, L) != SMOE_OK)
    return report_error(SMOE_E_UNSUPPORTED, "expert shape [%u, %u] has no canonical blob layout",
                        d[0].rows, v->h.d_model);
  return SMOE_OK;
}

// Entry i's blob in canonical layout into host memory dst (padded size).
int assemble(const smoe_vault* v, uint32_t i, const smoe_expert_layout& L, uint8_t* dst) {
  const smoe_expert_entry& e = v->entries[i];
  const smoe_tensor_desc* d = &v->descs[(uint64_t)i * 3];
  const smoe_tensor_layout* t[3] = {&L.gate, &L.up, &L.down};
  bool same = true;
  for (int k = 0; k < 3; ++k)
    same = same && d[k].packed_offset == t[k]->codes_offset && d[k].scales_offset == t[k]->scales_offset;
  memset(dst + L.raw_size, 0, L.padded_size - L.raw_size);
  if (same) {
    if (!read_at(v->fd, dst, L.raw_size, e.byte_offset))
      return report_error(SMOE_E_IO, "reading expert blob failed");
    return SMOE_OK;
  }
  for (int k = 0; k < 3; ++k) {
    if (!read_at(v->fd, dst + t[k]->codes_offset, t[k]->codes_bytes, e.byte_offset + d[k].packed_offset) ||
        !read_at(v->fd, dst + t[k]->scales_offset, t[k]->scales_bytes, e.byte_offset + d[k].scales_offset))
      return report_error(SMOE_E_IO, "reading expert tensors failed");
  }
  return SMOE_OK;
}

int find_index(const smoe_vault* v, uint32_t layer, uint32_t expert, uint32_t* i) {
  auto it = v->index.find(key_of(layer, expert));
  if (it == v->index.end())
    return report_error(SMOE_E_NOT_FOUND, "no expert (%u, %u) in the vault", layer, expert);
  *i = it->second;
  return SMOE_OK;
}

// Entries of layer_id as [first, first + count); they must be experts
// 0..count-1 of one shape for a bank.
int layer_range(const smoe_vault* v, uint32_t layer, uint32_t* first, uint32_t* count,
                smoe_expert_layout* L) {
  uint32_t i0;
  if (v->index.find(key_of(layer, 0)) == v->index.end()) {
    for (const auto& e : v->entries)
      if (e.layer_id == layer)
        return report_error(SMOE_E_UNSUPPORTED, "layer %u does not start at expert 0", layer);
    return report_error(SMOE_E_NOT_FOUND, "no layer %u in the vault", layer);
  }
  i0 = v->index.find(key_of(layer, 0))->second;
  uint32_t n = 0;
  while (i0 + n < v->entries.size() && v->entries[i0 + n].layer_id == layer) {
    if (v->entries[i0 + n].expert_id != n)
      return report_error(SMOE_E_UNSUPPORTED, "layer %u experts are not numbered 0..n-1", layer);
    if (v->descs[(uint64_t)(i0 + n) * 3].rows != v->descs[(uint64_t)i0 * 3].rows)
      return report_error(SMOE_E_UNSUPPORTED, "layer %u experts differ in shape", layer);
    ++n;
  }
  if (n > SMOE_MAX_EXPERTS)
    return report_error(SMOE_E_UNSUPPORTED, "layer %u has %u experts (at most %d per bank)", layer,
                        n, SMOE_MAX_EXPERTS);
  int rc = canonical(v, i0, L);
  if (rc) return rc;
  *first = i0;
  *count = n;
  return SMOE_OK;
}

}  // namespace

extern "C" {

void smoe_arch_block_init(smoe_arch_block* a) {
  if (!a) return;
  memset(a, 0, sizeof *a);
  memcpy(a->magic, kSarc, 4);
  a->block_version = 1;
  a->block_size = SMOE_SARC_SIZE;
  a->rms_norm_eps = 1e-6f;
}

int smoe_vault_plan(const smoe_vault_spec* spec, smoe_vault_header* header, uint64_t* file_size) {
  if (!header || !file_size) return report_error(SMOE_E_ARG, "null output");
  Plan p;
  int rc = make_plan(spec, &p, false);
  if (rc) return rc;
  *header = p.h;
  *file_size = p.file_size;
  return report_ok();
}

int smoe_vault_create(const char* path, const smoe_vault_spec* spec, smoe_vault_writer** out) {
  if (!out || !path) return report_error(SMOE_E_ARG, "null path or output");
  *out = nullptr;
  smoe_vault_writer* w = new (std::nothrow) smoe_vault_writer;
  if (!w) return report_error(SMOE_E_ARG, "out of host memory");
  int rc = make_plan(spec, &w->plan, true);
  if (rc) {
    delete w;
    return rc;
  }
  w->layer_ids.assign(spec->layer_ids, spec->layer_ids + spec->num_moe_layers);
  w->written.assign(w->plan.entries.size(), 0);
  w->fd = open(path, O_CREAT | O_TRUNC | O_WRONLY | O_CLOEXEC, 0644);
  if (w->fd < 0) {
    delete w;
    return report_error(SMOE_E_IO, "cannot create %s: %s", path, strerror(errno));
  }
  const Plan& p = w->plan;
  const uint64_t n = p.entries.size();
  bool good = write_at(w->fd, &p.h, sizeof p.h, 0) &&
              write_at(w->fd, p.entries.data(), n * sizeof(smoe_expert_entry), SMOE_VAULT_TABLE_OFFSET) &&
              write_at(w->fd, p.descs.data(), n * 3 * sizeof(smoe_tensor_desc),
                       SMOE_VAULT_TABLE_OFFSET + n * sizeof(smoe_expert_entry));
  if (good && p.h.version == 2) good = write_at(w->fd, &p.arch, sizeof p.arch, p.h.reserved_ext);
  // zero padding and not-yet-written blobs read as zero
  if (good) good = ftruncate(w->fd, (off_t)p.file_size) == 0;
  if (!good) {
    const int err = errno;
    close(w->fd);
    delete w;
    return report_error(SMOE_E_IO, "writing %s failed: %s", path, strerror(err));
  }
  *out = w;
  return report_ok();
}

int smoe_vault_put_expert(smoe_vault_writer* w, uint32_t layer_id, uint32_t expert_id,
                          const void* blob, uint64_t nbytes, int location, void* hip_stream) {
  if (!w || !blob) return report_error(SMOE_E_ARG, "null writer or blob");
  if (location != SMOE_MEM_HOST && location != SMOE_MEM_DEVICE)
    return report_error(SMOE_E_ARG, "unknown memory location %d", location);
  const Plan& p = w->plan;
  if (nbytes < p.L.raw_size)
    return report_error(SMOE_E_ARG, "blob holds %llu bytes, the raw size is %llu",
                        (unsigned long long)nbytes, (unsigned long long)p.L.raw_size);
  auto it = std::lower_bound(w->layer_ids.begin(), w->layer_ids.end(), layer_id);
  const uint32_t E = p.h.max_experts_per_layer;
  if (it == w->layer_ids.end() || *it != layer_id || expert_id >= E)
    return report_error(SMOE_E_NOT_FOUND, "expert (%u, %u) is not in this vault", layer_id, expert_id);
  const uint64_t i = (uint64_t)(it - w->layer_ids.begin()) * E + expert_id;
  const void* src = blob;
  if (location == SMOE_MEM_DEVICE) {
    int rc = w->st.ensure(p.L.raw_size);
    if (rc) return rc;
    hipError_t e = hipMemcpyAsync(w->st.buf[0], blob, p.L.raw_size, hipMemcpyDeviceToHost,
                                  (hipStream_t)hip_stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)hip_stream);
    if (e != hipSuccess) return hip_fail(e, "device blob copy");
    src = w->st.buf[0];
  }
  if (!write_at(w->fd, src, p.L.raw_size, p.entries[i].byte_offset))
    return report_error(SMOE_E_IO, "writing expert (%u, %u) failed: %s", layer_id, expert_id,
                        strerror(errno));
  w->written[i] = 1;
  return report_ok();
}

int smoe_vault_finish(smoe_vault_writer* w) {
  if (!w) return report_ok();
  uint64_t missing = 0;
  for (uint8_t b : w->written) missing += b ? 0 : 1;
  const bool closed = close(w->fd) == 0;
  delete w;
  if (missing)
    return report_error(SMOE_E_ARG, "%llu experts were never written", (unsigned long long)missing);
  if (!closed) return report_error(SMOE_E_IO, "closing the vault failed");
  return report_ok();
}

int smoe_vault_open(const char* path, smoe_vault** out) {
  if (!out || !path) return report_error(SMOE_E_ARG, "null path or output");
  *out = nullptr;
  smoe_vault* v = new (std::nothrow) smoe_vault;
  if (!v) return report_error(SMOE_E_IO, "out of host memory");
  v->fd = open(path, O_RDONLY | O_CLOEXEC);
  if (v->fd < 0) {
    delete v;
    return report_error(SMOE_E_IO, "cannot open %s: %s", path, strerror(errno));
  }
  struct stat sb;
  int rc = SMOE_OK;
  if (fstat(v->fd, &sb) != 0) {
    rc = report_error(SMOE_E_IO, "cannot stat %s", path);
  } else {
    v->size = (uint64_t)sb.st_size;
    if (v->size < sizeof v->h)
      rc = report_error(SMOE_E_FORMAT, "file shorter than the 64-byte header");
    else if (!read_at(v->fd, &v->h, sizeof v->h, 0))
      rc = report_error(SMOE_E_IO, "reading the header failed");
    else
      rc = validate(v);
  }
  if (rc) {
    close(v->fd);
    delete v;
    return rc;
  }
  *out = v;
  return report_ok();
}

void smoe_vault_close(smoe_vault* v) {
  if (!v) return;
  close(v->fd);
  delete v;
}

int smoe_vault_get_header(const smoe_vault* v, smoe_vault_header* header, smoe_arch_block* arch) {
  if (!v || !header) return report_error(SMOE_E_ARG, "null vault or header");
  *header = v->h;
  if (arch) *arch = v->arch;
  return report_ok();
}

int smoe_vault_find(const smoe_vault* v, uint32_t layer_id, uint32_t expert_id,
                    smoe_expert_entry* entry, smoe_tensor_desc* descs3) {
  if (!v) return report_error(SMOE_E_ARG, "null vault");
  uint32_t i;
  int rc = find_index(v, layer_id, expert_id, &i);
  if (rc) return rc;
  if (entry) *entry = v->entries[i];
  if (descs3) memcpy(descs3, &v->descs[(uint64_t)i * 3], 3 * sizeof(smoe_tensor_desc));
  return report_ok();
}

int smoe_vault_layer_desc(const smoe_vault* v, uint32_t layer_id, smoe_layer_desc* out) {
  if (!v || !out) return report_error(SMOE_E_ARG, "null vault or output");
  uint32_t first, count;
  smoe_expert_layout L;
  int rc = layer_range(v, layer_id, &first, &count, &L);
  if (rc) return rc;
  memset(out, 0, sizeof *out);
  out->d_model = v->h.d_model;
  out->ffn_dim = L.gate.rows;
  out->num_experts = count;
  out->bits = v->h.bits;
  out->group_size = SMOE_GROUP_SIZE;
  out->scale_dtype = SMOE_SCALE_F16;
  out->blob_stride = L.padded_size;
  return report_ok();
}

int smoe_vault_read_expert(smoe_vault* v, uint32_t layer_id, uint32_t expert_id, void* dst,
                           uint64_t nbytes, int location, void* hip_stream) {
  if (!v || !dst) return report_error(SMOE_E_ARG, "null vault or destination");
  if (location != SMOE_MEM_HOST && location != SMOE_MEM_DEVICE)
    return report_error(SMOE_E_ARG, "unknown memory location %d", location);
  uint32_t i;
  smoe_expert_layout L;
  int rc = find_index(v, layer_id, expert_id, &i);
  if (!rc) rc = canonical(v, i, &L);
  if (rc) return rc;
  if (nbytes < L.padded_size)
    return report_error(SMOE_E_ARG, "destination holds %llu bytes, the blob needs %llu",
                        (unsigned long long)nbytes, (unsigned long long)L.padded_size);
  if (location == SMOE_MEM_HOST) {
    rc = assemble(v, i, L, (uint8_t*)dst);
    return rc ? rc : report_ok();
  }
  rc = v->st.ensure(L.padded_size);
  if (!rc) rc = v->st.wait_all();
  if (!rc) rc = assemble(v, i, L, (uint8_t*)v->st.buf[0]);
  if (rc) return rc;
  hipError_t e = hipMemcpyAsync(dst, v->st.buf[0], L.padded_size, hipMemcpyHostToDevice,
                                (hipStream_t)hip_stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)hip_stream);
  return e == hipSuccess ? report_ok() : hip_fail(e, "blob copy to the device");
}

int smoe_vault_read_layer(smoe_vault* v, uint32_t layer_id, void* dst, uint64_t nbytes,
                          int location, void* hip_stream) {
  if (!v || !dst) return report_error(SMOE_E_ARG, "null vault or destination");
  if (location != SMOE_MEM_HOST && location != SMOE_MEM_DEVICE)
    return report_error(SMOE_E_ARG, "unknown memory location %d", location);
  uint32_t first, count;
  smoe_expert_layout L;
  int rc = layer_range(v, layer_id, &first, &count, &L);
  if (rc) return rc;
  if (nbytes / L.padded_size < count)
    return report_error(SMOE_E_ARG, "destination holds %llu bytes, the layer needs %llu",
                        (unsigned long long)nbytes, (unsigned long long)count * L.padded_size);
  uint8_t* base = (uint8_t*)dst;
  if (location == SMOE_MEM_HOST) {
    for (uint32_t j = 0; j < count; ++j) {
      rc = assemble(v, first + j, L, base + (uint64_t)j * L.padded_size);
      if (rc) return rc;
    }
    return report_ok();
  }
  rc = v->st.ensure(L.padded_size);
  if (rc) return rc;
  const hipStream_t s = (hipStream_t)hip_stream;
  for (uint32_t j = 0; j < count; ++j) {
    const int b = j & 1;
    rc = v->st.wait(b);
    if (!rc) rc = assemble(v, first + j, L, (uint8_t*)v->st.buf[b]);
    if (rc) {
      v->st.wait_all();
      return rc;
    }
    hipError_t e = hipMemcpyAsync(base + (uint64_t)j * L.padded_size, v->st.buf[b], L.padded_size,
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(v->st.done[b], s);
    if (e != hipSuccess) {
      v->st.wait_all();
      return hip_fail(e, "blob copy to the device");
    }
    v->st.pending[b] = true;
  }
  rc = v->st.wait_all();
  return rc ? rc : report_ok();
}

}  // extern "C"
