"""MHLA forward on MI355X (placeholder, binding follows)."""
