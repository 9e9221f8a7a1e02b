/*
 * smoe_vault.h -- C ABI of the .smoe vault reader and writer (host code in
 * libsmoe.so; the blobs go to or come from device or host memory).
 *
 * Source (page title, sections): ".smoe Binary Format" -- Immutable
 * Encoding (little-endian integers, offsets from the start of the file,
 * blobs on 16,384-byte boundaries), File Architecture (header, expert table,
 * tensor descriptors, arch block, zero padding, blobs), File Header, Version
 * acceptance, Arch Block "SARC", Expert Table Entry, Flash Lookup, Tensor
 * Descriptor, Expert Blob Architecture, C++ Struct Mirror (the three fixed
 * struct sizes).
 *
 * The structs below are the on-disk records byte for byte (packed, no
 * padding; little-endian hosts only). Conventions of smoe.h apply: status
 * codes, smoe_last_error(), no exception crosses the ABI, host-side checks
 * before any I/O or GPU work.
 *
 * What a reader accepts (every check is made by smoe_vault_open; a file that
 * fails one is refused with SMOE_E_FORMAT and a message naming the check):
 *  header   magic 53 4D 4F 45 DE EA 00 01; version 1 or 2; table_offset 64;
 *           group_size 64; bits 2 or 4; data_offset a multiple of 16,384,
 *           past the metadata and inside the file; total_experts >= 1;
 *           num_moe_layers = the number of distinct layer ids in the table;
 *           max_experts_per_layer = the most entries any layer has.
 *  v1       reserved_ext == 0 (no arch block).
 *  v2       reserved_ext a multiple of 64, at or after the end of the
 *           descriptors, with the 128-byte block ending at or before
 *           data_offset; the block has magic "SARC", block_version 1,
 *           block_size 128, activation 0 (SiLU / SwiGLU), 1 <= moe_top_k <= 16,
 *           head_dim <= 256, num_kv_heads >= 1 dividing num_heads, reserved
 *           bytes zero.
 *  table    entries sorted by (layer_id, expert_id), strictly ascending;
 *           group_size = the header's; reserved bytes zero; byte_offset a
 *           multiple of 16,384 at or after data_offset; padded_size =
 *           raw_size rounded up to 16,384; blobs inside the file and not
 *           overlapping; num_groups = the three tensors' ceil(rows*cols/64).
 *  desc     three per entry, tensor_type 0, 1, 2 (gate, up, down) in that
 *           order; ndim 2; reserved_0 zero; gate and up [ffn, d_model], down
 *           [d_model, ffn] with d_model the header's and ffn >= 1;
 *           packed_size ceil(rows*cols*bits/8); scales_size
 *           ceil(rows*cols/64)*2 (fp16 scales); the six byte ranges inside
 *           raw_size and not overlapping.
 */
#ifndef SMOE_VAULT_H_
#define SMOE_VAULT_H_

#include <stdint.h>

#include "smoe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SMOE_E_FORMAT (-6)    /* not a valid .smoe vault (see the checks above) */
#define SMOE_E_IO (-7)        /* open, read, write or size query failed          */
#define SMOE_E_NOT_FOUND (-8) /* no such (layer, expert) or layer in the vault   */

#define SMOE_MEM_HOST 0   /* pointer is ordinary host memory */
#define SMOE_MEM_DEVICE 1 /* pointer is device memory        */

#define SMOE_VAULT_VERSION 2       /* version this library writes by default */
#define SMOE_VAULT_TABLE_OFFSET 64 /* the expert table follows the header   */
#define SMOE_SARC_SIZE 128

#pragma pack(push, 1)

/* File Header, 64 bytes at offset 0. */
typedef struct smoe_vault_header {
  uint8_t magic[8];               /* 53 4D 4F 45 DE EA 00 01                 */
  uint32_t version;               /* 1 or 2                                  */
  uint32_t num_moe_layers;        /* distinct layer ids in the table          */
  uint32_t max_experts_per_layer; /* largest expert count of a layer          */
  uint32_t total_experts;         /* table entries                            */
  uint64_t table_offset;          /* 64                                       */
  uint64_t data_offset;           /* first blob, multiple of 16,384           */
  uint32_t group_size;            /* 64                                       */
  uint32_t bits;                  /* 2 or 4                                   */
  uint32_t d_model;               /* hidden size                              */
  uint32_t vocab_size;            /* stored as written                        */
  uint32_t ffn_dim;               /* dense / shared FFN size, stored as written */
  uint32_t reserved_ext;          /* v2: file offset of the arch block; v1: 0 */
} smoe_vault_header;

/* Arch Block "SARC", 128 bytes at header.reserved_ext (v2). */
typedef struct smoe_arch_block {
  uint8_t magic[4];               /* "SARC"                                   */
  uint32_t block_version;         /* 1                                        */
  uint32_t block_size;            /* 128                                      */
  uint32_t flags;                 /* bit 0 norm_topk_prob, bit 1 has_qk_norm,
                                     bit 2 has_dense_layer_0                  */
  float rope_theta;
  uint32_t num_heads;
  uint32_t num_kv_heads;
  uint32_t head_dim;
  uint32_t moe_top_k;
  uint32_t moe_ffn_dim;
  uint32_t dense_ffn_dim;
  uint32_t shared_expert_ffn_dim; /* 0 = none                                 */
  uint32_t activation;            /* 0 = SiLU / SwiGLU                        */
  uint32_t num_hidden_layers;
  float rms_norm_eps;
  char model_type[24];            /* NUL-padded                               */
  uint8_t reserved[44];           /* zero                                     */
} smoe_arch_block;

/* Expert Table Entry, 48 bytes; total_experts of them from offset 64. */
typedef struct smoe_expert_entry {
  uint32_t layer_id;
  uint32_t expert_id;
  uint64_t byte_offset;           /* file offset of the blob                  */
  uint64_t raw_size;              /* data bytes before padding                */
  uint64_t padded_size;           /* raw_size rounded up to 16,384            */
  uint32_t group_size;            /* = header.group_size                      */
  uint64_t num_groups;            /* groups over the three tensors            */
  uint8_t reserved[4];            /* zero                                     */
} smoe_expert_entry;

/* Tensor Descriptor, 44 bytes; three per entry (gate, up, down) right after
 * the table. Offsets are relative to the expert's blob. */
typedef struct smoe_tensor_desc {
  uint8_t tensor_type;            /* 0 gate_proj, 1 up_proj, 2 down_proj      */
  uint8_t ndim;                   /* 2                                        */
  uint8_t reserved_0[2];          /* zero                                     */
  uint32_t rows, cols;            /* the weight's [out, in] shape             */
  uint64_t packed_offset, packed_size;
  uint64_t scales_offset, scales_size; /* fp16 scales                         */
} smoe_tensor_desc;

#pragma pack(pop)

#ifdef __cplusplus
static_assert(sizeof(smoe_vault_header) == 64, "header is 64 bytes");
static_assert(sizeof(smoe_arch_block) == 128, "arch block is 128 bytes");
static_assert(sizeof(smoe_expert_entry) == 48, "table entry is 48 bytes");
static_assert(sizeof(smoe_tensor_desc) == 44, "tensor descriptor is 44 bytes");
#else
_Static_assert(sizeof(smoe_vault_header) == 64, "header is 64 bytes");
_Static_assert(sizeof(smoe_arch_block) == 128, "arch block is 128 bytes");
_Static_assert(sizeof(smoe_expert_entry) == 48, "table entry is 48 bytes");
_Static_assert(sizeof(smoe_tensor_desc) == 44, "tensor descriptor is 44 bytes");
#endif

/* ---------------------------------------------------------------- writer */

/* What to write. Every expert of the vault has the same shape (gate and up
 * [moe_ffn_dim, d_model], down [d_model, moe_ffn_dim]), and its blob is the
 * canonical layout smoe_expert_layout_of(d_model, moe_ffn_dim, bits,
 * SMOE_SCALE_F16) gives: the three tensors woven back to back, fp16 scales.
 * The table lists layer_ids[0..n-1] x experts 0..experts_per_layer-1 in that
 * order; blobs follow in table order from data_offset, padded_size apart.
 * Metadata placement: table at 64, descriptors right after it, the arch block
 * (v2) at the next multiple of 64, data_offset the next multiple of 16,384. */
typedef struct smoe_vault_spec {
  uint32_t version;               /* 1 (no arch block) or 2                   */
  uint32_t bits;                  /* 2 or 4                                   */
  uint32_t d_model;               /* multiple of 64                           */
  uint32_t moe_ffn_dim;           /* multiple of 64                           */
  uint32_t vocab_size;            /* header field, stored as given            */
  uint32_t ffn_dim;               /* header field, stored as given            */
  uint32_t num_moe_layers;        /* >= 1                                     */
  uint32_t experts_per_layer;     /* >= 1                                     */
  const uint32_t* layer_ids;      /* host [num_moe_layers], strictly ascending */
  const smoe_arch_block* arch;    /* host; required for v2 (it must pass the
                                     reader's arch checks), NULL for v1       */
} smoe_vault_spec;

typedef struct smoe_vault_writer smoe_vault_writer;

/* A block with magic "SARC", block_version 1, block_size 128, rms_norm_eps
 * 1e-6 and every other field zero (activation 0 = SiLU). */
void smoe_arch_block_init(smoe_arch_block* arch);

/* The metadata a spec produces, without touching a file: the header and the
 * file size. Errors: SMOE_E_ARG for a spec the writer would refuse. */
int smoe_vault_plan(const smoe_vault_spec* spec, smoe_vault_header* header,
                    uint64_t* file_size);

/* Create (truncate) the file at path, write header, table, descriptors, arch
 * block and zero padding, and size the file so that unwritten blob bytes read
 * as zero. *out owns the open file until smoe_vault_finish.
 * Errors: SMOE_E_ARG (spec), SMOE_E_IO. */
int smoe_vault_create(const char* path, const smoe_vault_spec* spec,
                      smoe_vault_writer** out);

/* Write one expert's blob: the first raw_size bytes of blob (canonical
 * layout, at least raw_size bytes long), then zeros up to padded_size.
 * location SMOE_MEM_HOST or SMOE_MEM_DEVICE (then the bytes are copied on
 * hip_stream into a pinned staging buffer the writer owns, and the call waits
 * for that copy). Writing an expert again overwrites it. Not thread-safe per
 * writer. Errors: SMOE_E_ARG (null, unknown location, blob shorter than the
 * raw size), SMOE_E_NOT_FOUND (layer or expert not in the spec), SMOE_E_HIP,
 * SMOE_E_IO. */
int smoe_vault_put_expert(smoe_vault_writer* writer, uint32_t layer_id, uint32_t expert_id,
                          const void* blob, uint64_t nbytes, int location, void* hip_stream);

/* Close the file and free the writer (always, also on error). Errors:
 * SMOE_E_ARG if some expert was never written (the file stays, with zero
 * blobs there), SMOE_E_IO if closing failed. NULL is a no-op. */
int smoe_vault_finish(smoe_vault_writer* writer);

/* ---------------------------------------------------------------- reader */

typedef struct smoe_vault smoe_vault;

/* Open and validate a vault: reads the header, table, descriptors and arch
 * block into host memory (the blobs stay on disk) and builds the
 * (layer, expert) lookup. Errors: SMOE_E_ARG (null), SMOE_E_IO,
 * SMOE_E_FORMAT. */
int smoe_vault_open(const char* path, smoe_vault** out);

/* Close the file and free the handle (NULL is a no-op). */
void smoe_vault_close(smoe_vault* vault);

/* Copies of the header and (nullable) the arch block; for a v1 vault the
 * arch block comes back all zero. Errors: SMOE_E_ARG (null vault or header). */
int smoe_vault_get_header(const smoe_vault* vault, smoe_vault_header* header,
                          smoe_arch_block* arch);

/* Flash lookup: the table entry and (nullable) its three descriptors for
 * (layer_id, expert_id). Errors: SMOE_E_ARG, SMOE_E_NOT_FOUND. */
int smoe_vault_find(const smoe_vault* vault, uint32_t layer_id, uint32_t expert_id,
                    smoe_expert_entry* entry, smoe_tensor_desc* descs3);

/* The smoe_layer_desc of one MoE layer's bank as smoe_vault_read_layer
 * fills it: num_experts = the layer's entries, which must be experts
 * 0..n-1 of one shape (SMOE_E_UNSUPPORTED otherwise, or when the shape is
 * not one smoe_load_blobs takes); fp16 scales; blob_stride = the canonical
 * padded size; no shared expert. Errors: SMOE_E_ARG, SMOE_E_NOT_FOUND,
 * SMOE_E_UNSUPPORTED. */
int smoe_vault_layer_desc(const smoe_vault* vault, uint32_t layer_id, smoe_layer_desc* out);

/* One expert's blob in canonical layout (tensors moved from the descriptors'
 * offsets to the canonical ones when they differ), zero-filled up to the
 * canonical padded size, into dst (location SMOE_MEM_HOST or
 * SMOE_MEM_DEVICE). nbytes >= the canonical padded size. A device copy runs
 * on hip_stream from a pinned staging buffer the handle owns; the call
 * returns once it is complete. Not thread-safe per handle.
 * Errors: SMOE_E_ARG, SMOE_E_NOT_FOUND, SMOE_E_UNSUPPORTED (shape without a
 * canonical layout), SMOE_E_IO, SMOE_E_HIP. */
int smoe_vault_read_expert(smoe_vault* vault, uint32_t layer_id, uint32_t expert_id, void* dst,
                           uint64_t nbytes, int location, void* hip_stream);

/* A whole layer as the bank smoe_load_blobs takes: expert e at
 * dst + e * desc.blob_stride for the desc smoe_vault_layer_desc returns;
 * nbytes >= num_experts * blob_stride. Device copies are double-buffered
 * (the next blob is read from disk while the previous one is copied); the
 * call returns once every copy is complete. Errors as
 * smoe_vault_read_expert. */
int smoe_vault_read_layer(smoe_vault* vault, uint32_t layer_id, void* dst, uint64_t nbytes,
                          int location, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_VAULT_H_ */
